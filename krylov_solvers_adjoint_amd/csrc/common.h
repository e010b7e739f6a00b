// Internal definitions shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
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

// Report a failed kernel launch (call after launching, inside a function
// that returns sla_status).
#define LAUNCH_CHECK()                                                         \
  do {                                                                         \
    hipError_t e_ = hipGetLastError();                                         \
    if (e_ != hipSuccess) {                                                    \
      ::sla::set_error("kernel launch failed: %s (%s:%d)",                     \
                       hipGetErrorString(e_), __FILE__, __LINE__);             \
      return SLA_ERR_DEVICE;                                                   \
    }                                                                          \
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
constexpr int kWave = 64;
constexpr int kBlock = 256;        // workgroup of the set-up kernels (4 waves)
constexpr int kIterBlock = 1024;   // workgroup of most solver kernels (16 waves)
constexpr int kWaves = kIterBlock / kWave;
// two solver workgroups per CU: 8 waves on each of its 4 SIMDs, which caps a
// kernel at 64 VGPRs
constexpr int kWavesPerEu = 2 * kWaves / 4;
constexpr int kTileRows = 64;      // rows per wave tile: one row per lane
constexpr int kXcds = 8;           // MI355X: 8 XCDs, workgroups dealt round-robin
// Staged (value, column) slots per wave tile: 16 waves x 336 slots x 12 B
// stays under 64 KiB per workgroup, so two solver workgroups fit the LDS of a
// CU; a 64-row tile of a 5-point stencil has at most 320 slots.
constexpr int kWaveCap = 336;
constexpr int kStageLoads = (kWaveCap + kWave - 1) / kWave;  // staged slots per lane
constexpr int kPartSets = 7;       // partial-sum arrays per system (see Ctx)
constexpr int kMaxBand = 8;        // most distinct column offsets of a banded pattern
constexpr int64_t kMaxBandSpan = int64_t(1) << 27;  // widest band (largest - smallest offset)
constexpr int kPanelTiles = 64;    // widest column block of the panel tile order
// line walk: workgroups of 8 waves, two per CU (4 waves per SIMD, 128
// registers each)
constexpr int kLineWaves = 8;
constexpr int kLineWavesPerEu = 2 * kLineWaves / 4;
// a line walk whose waves walk at least this many lines per chunk keeps two
// tiles of loads in flight (shorter walks do better with one)
constexpr int64_t kPipeLines = 12;
// ... on matrices of at most this many rows (beyond, the walk streams from
// HBM and the simpler loop is as fast)
constexpr int64_t kPipeMaxRows = int64_t(1) << 26;
// a line walk needs at least 16 tile columns per line
constexpr int64_t kMinWalkLine = int64_t(kIterBlock / kWave - 1) * kTileRows + 1;
// a 64-row tile whose columns span more than this is "wide" (the span of a
// 5-point stencil tile on a 13000-point grid line is ~26000)
constexpr int64_t kLocalSpan = int64_t(1) << 17;
// solves of at most this many unknowns (over the batch) run one solver
// workgroup per CU unless the handle asks otherwise
constexpr int64_t kSmallSolve = int64_t(1) << 21;
// the one-workgroup CG solver takes systems of up to this many unknowns
// (beyond, one CU per system is slower than the grid)
constexpr int64_t kOneGroupMaxN = 2048;

// Column offsets j - i of a banded pattern, ascending: row i's slots are the
// columns i + off[t] for the bits t set in its mask byte.
struct BandOffsets {
  int32_t count;
  int32_t off[kMaxBand];
};

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
  ST_BREAKDOWN = SLA_ERR_BREAKDOWN,
  // the resident grid loop: a wait for the other workgroups exceeded its
  // poll limit (every workgroup then leaves the loop); no sla_status value
  ST_GRID_TIMEOUT = 100,
};

// Per-system CG scalars, resident on the device for the whole solve.  An
// iteration is two kernels, the SpMV step and the residual step.  Every field
// is written by one of them (one thread of workgroup 0) and read only by the
// other or by the host, so no workgroup ever reads a field that another
// workgroup of the same launch may be writing.
struct alignas(64) Scal {
  double rr[2];     // r_k . r_k, by parity of k          (SpMV step writes)
  double rz[2];     // r_k . z_k (Jacobi), by parity of k  (SpMV step writes)
  double alpha[2];  // alpha_k, by parity of k               (residual step writes)
  double bb;        // b . b                                (set-up)
  double stop;      // (tol * tol) * bb                     (set-up)
  double rr_final;  // r . r when the system stopped        (the stopping step)
  int64_t ka;       // index of the next SpMV step          (residual step writes)
  int64_t kr;       // index of the next residual step      (SpMV step writes)
  int64_t it;       // completed iterations when stopped    (the stopping step)
  int64_t maxit;    //                                      (set-up)
  int32_t state_a;  // state as set by SpMV steps           (SpMV step writes)
  int32_t state_r;  // state as set by residual steps       (residual step writes)
};

// Everything the solver kernels touch, resident in device memory so that a
// captured graph stays valid while the caller's x / b / values change.  The
// systems' Scal records follow it in the same allocation (see scal_of).
struct alignas(64) Ctx {
  const void* rowptr;
  const int32_t* col;
  const double* vals;   // [batch][nnz]
  double* x;            // [batch][n] solution (lambda for the adjoint)
  const double* b;      // [batch][n] right-hand side
  double* r;            // [batch][n]
  // Jacobi preconditioning (M = diag(A)): z = r / d, the search direction is
  // built from z; without it `rd` is r and `diag`, `z`, `bad` are unused
  const double* diag;   // [batch][n] the diagonal d, extracted at set-up
  double* z;            // [batch][n]
  const double* rd;     // [batch][n] source of the search direction: z or r
  int* bad;             // [batch] set when a diagonal entry is not > 0
  int32_t jacobi;
  double* p[2];         // [batch][n] search direction, double-buffered
  double* q;            // [batch][n] A p
  // [batch][kPartSets][grid] one partial per workgroup:
  //   set 0/1: r.r by parity of k, set 2/3: p.Ap by parity of k, set 4: b.b,
  //   set 5/6: r.z by parity of k (Jacobi)
  double* part;
  Scal* scal;           // [batch]
  double* hist;         // [batch][hist_cap][3] alpha, beta, rr or nullptr
  int* n_running;       // systems still iterating
  int64_t hist_cap;
  int64_t n;
  int64_t nnz;
  int64_t batch;
  int64_t tiles;        // ceil(n / kTileRows)
  int32_t grid;         // workgroups per system in the solver kernels
  int32_t wave_cap;     // staged slots per wave tile (>= 1)
  const uint8_t* mask;  // [n] band masks, or nullptr (plain CSR)
  BandOffsets band;
  int32_t panel;        // tiles per band span (0: rows in plain order)
  int32_t pblock;       // tiles per column block of the panel order
  int64_t line;         // grid line length of a line-walk band (0: none)
  int32_t line_chunks;  // line chunks per XCD in the line walk
  // the line walk applies x's deferred updates two at a time: the SpMV step
  // of an even k >= 2 adds alpha_{k-2} p_{k-2} and alpha_{k-1} p_{k-1}, odd
  // steps leave x alone (the other kernels add alpha_{k-1} p_{k-1} at every k)
  int32_t xpair;
};
static_assert(sizeof(Ctx) % alignof(Scal) == 0, "Scal records follow the context");

// System s's scalars: the records right after the context, so that a kernel
// can load them in the same round trip as the context's own fields (through
// `scal` it would wait for the context first).
__host__ __device__ __forceinline__ Scal* scal_of(const Ctx* c, int64_t s) {
  return reinterpret_cast<Scal*>(const_cast<Ctx*>(c) + 1) + s;
}

// The context and one system's record in one round trip (see load_ctx).
constexpr uint32_t kCtxWords = sizeof(Ctx) / 8;
constexpr uint32_t kScalWords = sizeof(Scal) / 8;
struct CtxWords {
  uint32_t lo, hi;
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Global-memory view of a pointer.  Pointers read from the device-resident
// context are generic to the compiler, which then emits flat loads; a flat
// load counts against both the vector-memory and the LDS counters, so every
// LDS access after it waits for it.  All buffers here are global memory.
#define SLA_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ SLA_GLOBAL T* gmem(T* p) {
  return (SLA_GLOBAL T*)(p);
}

// A value that is the same in every lane, moved to scalar registers (values
// that come from LDS or from vector loads live in vector registers).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return (uint64_t(hi) << 32) | lo;
}
// Ties uniform values to this point of the kernel: their scalar loads are
// issued before it.  Pinning all the context and record fields a kernel
// needs ahead of its first branch puts those loads under one wait; left to
// itself the compiler issues them a round trip apart, or sinks them past the
// branch, and each round trip costs the latency of the memory-side cache.
template <typename T>
__device__ __forceinline__ void pin1(const T& v) {
  __asm__ __volatile__("" : : "s"(v));
}
template <typename... T>
__device__ __forceinline__ void pin(const T&... v) {
  (pin1(v), ...);
}

__device__ __forceinline__ double uniform(double v) {
  return __longlong_as_double(int64_t(uniform_u64(uint64_t(__double_as_longlong(v)))));
}
__device__ __forceinline__ int64_t uniform(int64_t v) { return int64_t(uniform_u64(uint64_t(v))); }

// base[off] for a wave-uniform `base` and a non-negative offset whose byte
// offset fits in 32 bits.  The base is moved to scalar registers (it may sit
// in vector registers when the compiler cannot prove the context field it
// came from unclobbered) and hidden from reassociation by an empty asm, so
// the load takes the base in scalar registers and the offset in one vector
// register; otherwise the compiler folds a tile's base into a 64-bit
// per-lane address for every array and keeps those live across the loop.
// Every caller passes a base that is the same in all lanes of the wave.
template <typename T>
__device__ __forceinline__ uint64_t scalar_base(const SLA_GLOBAL T* p) {
  // readfirstlane returns int: both halves go through uint32_t before they
  // are widened, so the low half is zero- and not sign-extended
  uint64_t u = uniform_u64(reinterpret_cast<uint64_t>(p));
  asm("" : "+s"(u));
  return u;
}
template <typename T>
__device__ __forceinline__ T ld(const SLA_GLOBAL T* base, uint32_t off) {
  return *reinterpret_cast<const SLA_GLOBAL T*>(scalar_base(base) +
                                                uint64_t(off * uint32_t(sizeof(T))));
}
template <typename T>
__device__ __forceinline__ void st(SLA_GLOBAL T* base, uint32_t off, T v) {
  *reinterpret_cast<SLA_GLOBAL T*>(scalar_base(base) + uint64_t(off * uint32_t(sizeof(T)))) = v;
}

// Wait until every vector memory operation of this wave has completed
// (s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima).  Placed
// after a loop's prologue loads, it keeps the compiler from merging those
// pending loads into the loop head, where the wait for them would also wait
// for the stores of the previous iteration.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Index of this thread's wave in its workgroup, as a wave-uniform (scalar)
// value, so that everything derived from it stays in scalar registers.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
}
__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// The context and system s's record in one vector load: lane l loads 8-byte
// word l of the context (l < kCtxWords) or word l - kCtxWords of the record,
// and the kernel moves the fields it uses into scalar registers with
// readlane (no memory access).  Scalar loads of the same fields issue in
// dependent rounds (the compiler reuses scalar registers between them): four
// in the residual step, whose iteration at 10^6 unknowns this load shortens
// by about 0.5 us.  The pipelined line walk uses it too (fewer spills); the
// one-tile walk's rounds cost no more than this load (its context fields hit
// the scalar cache), and it keeps scalar loads.
__device__ __forceinline__ CtxWords load_ctx(const Ctx* c, int64_t s) {
  static_assert(kCtxWords + kScalWords <= kWave, "the context and a record fit one wave load");
  const uint32_t l = lane_id();
  const uint32_t lr = l - kCtxWords < kScalWords ? l - kCtxWords : 0u;
  const uint64_t* src = l < kCtxWords ? reinterpret_cast<const uint64_t*>(c) + l
                                      : reinterpret_cast<const uint64_t*>(scal_of(c, s)) + lr;
  const uint64_t w = *gmem(src);
  return CtxWords{uint32_t(w), uint32_t(w >> 32)};
}
// The field at byte offset `off` of the context, or (off >= sizeof(Ctx)) of
// the record, from the words of load_ctx.
template <typename T, uint32_t off>
__device__ __forceinline__ T ctx_get(const CtxWords& w) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte fields");
  static_assert(off % sizeof(T) == 0 && off / 8 < kCtxWords + kScalWords, "an aligned field");
  constexpr int word = int(off / 8);
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(w.hi), word))) << 32) |
                       uint32_t(__builtin_amdgcn_readlane(int(w.lo), word));
    return __builtin_bit_cast(T, u);
  } else {
    const uint32_t u = uint32_t(__builtin_amdgcn_readlane(int((off & 4u) ? w.hi : w.lo), word));
    return __builtin_bit_cast(T, u);
  }
}
#define SLA_CTX(w, T, field) ctx_get<T, uint32_t(offsetof(Ctx, field))>(w)
#define SLA_REC(w, T, field) ctx_get<T, uint32_t(sizeof(Ctx) + offsetof(Scal, field))>(w)
__device__ __forceinline__ BandOffsets ctx_band(const CtxWords& w) {
  static_assert(kMaxBand == 8, "one line per offset below");
  constexpr uint32_t o = uint32_t(offsetof(Ctx, band));
  BandOffsets b;
  b.count = ctx_get<int32_t, o>(w);
  b.off[0] = ctx_get<int32_t, o + 4>(w);
  b.off[1] = ctx_get<int32_t, o + 8>(w);
  b.off[2] = ctx_get<int32_t, o + 12>(w);
  b.off[3] = ctx_get<int32_t, o + 16>(w);
  b.off[4] = ctx_get<int32_t, o + 20>(w);
  b.off[5] = ctx_get<int32_t, o + 24>(w);
  b.off[6] = ctx_get<int32_t, o + 28>(w);
  b.off[7] = ctx_get<int32_t, o + 32>(w);
  return b;
}

// A double moved across lanes by a DPP pattern (two 32-bit moves); lanes
// without a source lane, or in rows the mask leaves out, read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xF, false);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum(double v) {
  // Sum over the 64 lanes by DPP moves (no lane permutes through LDS), one
  // fixed association order, the total in every lane: pairs (quad_perm
  // 1,0,3,2), quads (2,3,0,1), half rows (half mirror) and rows (mirror)
  // leave every lane of a 16-lane row with the row's sum; row 1 adds row 0's
  // and row 3 row 2's (broadcast of lane 15), rows 2 and 3 add lane 31's;
  // lane 63 then holds (r3 + r2) + (r1 + r0), read back into every lane.
  const int row = int(threadIdx.x & (kWave - 1)) >> 4;
  v = v + dpp_f64<0xB1>(v);
  v = v + dpp_f64<0x4E>(v);
  v = v + dpp_f64<0x141>(v);
  v = v + dpp_f64<0x140>(v);
  const double b15 = dpp_f64<0x142, 0xA>(v);
  v = (row & 1) ? v + b15 : v;
  const double b31 = dpp_f64<0x143, 0xC>(v);
  v = (row >= 2) ? v + b31 : v;
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), kWave - 1);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), kWave - 1);
  return __hiloint2double(hi, lo);
}

// Sum over a workgroup of NT threads, fixed order, result in every thread.
// `lds` holds NT / 64 doubles.
template <int NT>
__device__ __forceinline__ double block_sum_all(double v, double* lds) {
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) t = t + lds[w];
  __syncthreads();
  return t;
}

// The same sum without the closing barrier, for an `lds` area that the
// launch uses for no other sum (the barrier only protects an area's reuse).
template <int NT>
__device__ __forceinline__ double block_sum_once(double v, double* lds) {
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) t = t + lds[w];
  return t;
}

// Make a wave's LDS writes visible to its other lanes (a wave tile is owned
// by one wave, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tiles of wave `w` of workgroup `bid` (of `grid`, a multiple of kXcds): the
// tiles are split into kXcds contiguous ranges, one per XCD (workgroup i runs
// on XCD i % 8), and the waves of one XCD interleave over its range, so that
// at any time they work on neighbouring rows and share that XCD's L2.
struct TileWalk {
  int64_t first, stride, end;
};
__device__ __forceinline__ TileWalk wave_walk(int64_t tiles, int grid, int bid, int waves,
                                              int w) {
  const int xcd = bid % kXcds;
  const int per_xcd = grid / kXcds;
  const int slot = bid / kXcds;
  const int64_t lo = tiles * xcd / kXcds;
  const int64_t hi = tiles * (xcd + 1) / kXcds;
  return TileWalk{lo + int64_t(slot) * waves + w, int64_t(per_xcd) * waves, hi};
}

// Tile order of one XCD's range [lo, hi) for a banded pattern whose
// neighbours lie up to `panel` tiles away: the range is cut into panels of
// `panel` tiles, and position p walks column blocks of `pblock` tiles down
// all panels before moving to the next block, so a tile and its neighbours
// one panel up and down are in flight together and share the L2.  Returns -1
// for positions that fall past the end of a panel or of the range.
__device__ __forceinline__ int64_t panel_tile(int64_t p, int64_t lo, int64_t hi, int panel,
                                              int pblock) {
  // every quantity is below 2^31 (tiles of an int32-column matrix)
  const uint32_t V = uint32_t((hi - lo + panel - 1) / panel);
  const uint32_t per_blk = V * uint32_t(pblock);
  const uint32_t pp = uint32_t(p);
  const uint32_t blk = pp / per_blk;
  const uint32_t rem = pp - blk * per_blk;
  const uint32_t v = rem / uint32_t(pblock);
  const uint32_t u = blk * uint32_t(pblock) + (rem - v * uint32_t(pblock));
  if (u >= uint32_t(panel)) return -1;
  const int64_t t = lo + int64_t(v) * panel + u;
  return t < hi ? t : -1;
}

// Number of positions panel_tile walks for a range of `cnt` tiles.
__device__ __forceinline__ int64_t panel_positions(int64_t cnt, int panel, int pblock) {
  const int64_t V = (cnt + panel - 1) / panel;
  const int64_t nb = (panel + pblock - 1) / pblock;
  return nb * V * pblock;
}

}  // namespace sla

struct sla_csr_s;  // defined in handle.h
