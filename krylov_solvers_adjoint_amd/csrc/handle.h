// The matrix handle: pattern, bound values, and the solver workspace.
#pragma once

#include <map>
#include <utility>

#include "common.h"

namespace sla {
struct EigWork;  // Lanczos workspace (lanczos.hip)
struct BsWork;   // BiCGStab workspace (bicgstab.hip)
struct Reorder;  // locality ordering and the permuted matrix (reorder.hip)
}

struct sla_csr_s {
  int device = 0;
  int64_t n = 0;
  int64_t nnz = 0;
  int64_t nnz_coo = 0;
  sla_index rp_idx = SLA_I32;

  // pattern (owned)
  void* rowptr = nullptr;          // [n+1] int32 or int64
  int32_t* col = nullptr;          // [nnz]
  int64_t* perm = nullptr;         // [nnz_coo] COO triplet -> slot (COO only)
  uint32_t* sorted_idx = nullptr;  // [nnz_coo] triplet of each sorted position
  int64_t* grp = nullptr;          // [nnz+1] first sorted position of each slot

  // pattern analysis
  int64_t tiles = 0;           // ceil(n / kTileRows): 64-row wave tiles
  int64_t max_tile_nnz = 0;    // largest number of slots in one wave tile
  int32_t wave_cap = 0;        // slots staged per wave tile (>= 1 once analysed)
  // banded patterns (every column j = i + one of a few offsets): a mask
  // byte per row replaces the column array and per-row row pointers
  uint8_t* band_mask = nullptr;  // [n] or nullptr
  sla::BandOffsets band{};
  bool no_band = false;          // pattern analysis skips band detection
  int spmv_variant = SLA_SPMV_AUTO;  // SLA_SPMV_AUTO / _CSR / _BANDED / _SPLIT / _LINES
  int32_t panel = 0;             // panel order of the SpMV tiles (0 = rows in order)
  bool wide_cols = false;        // sampled tiles reach columns far apart
  int32_t pblock = 0;

  // bound values: the caller's array (sla_csr_set_values) or the handle's
  // own copy (sla_csr_load_values), [batch][nnz] in CSR slot order
  const double* vals = nullptr;
  int64_t batch = 0;
  double* vals_owned = nullptr;  // the handle's copy, [owned_batch][nnz]
  int64_t owned_batch = 0;

  // symmetry of the pattern (CG needs A^T = A): -1 not yet checked, 0 no, 1 yes
  int sym_pattern = -1;
  int* sym_flag = nullptr;  // device word of the symmetry checks

  // the transposed pattern, built on first use by the transposed product:
  // a handle of its own whose COO triplets are this pattern's slots with
  // rows and columns swapped, so that its sorted_idx maps each of its slots
  // to the slot of ours it transposes
  sla_csr_s* trans = nullptr;

  // workspace, sized for ws_cap systems (and part_cap partials); the last
  // solve ran ws_batch <= ws_cap of them
  int64_t ws_batch = 0;
  int64_t ws_cap = 0;
  int64_t part_cap = 0;
  int32_t grid = 0;            // iteration workgroups per system of ws_batch
  double* r = nullptr;
  double* p0 = nullptr;
  double* p1 = nullptr;
  double* q = nullptr;
  double* part = nullptr;      // [part_cap] >= kPartSets * ws_batch * grid
  sla::Scal* scal = nullptr;   // [ws_cap]
  int* n_running = nullptr;
  sla::Ctx* ctx_dev = nullptr;
  sla::Ctx* ctx_host = nullptr;      // pinned
  sla::Scal* scal_host = nullptr;    // pinned [ws_cap]
  int* poll_host = nullptr;          // pinned [2]
  hipEvent_t poll_ev[2] = {nullptr, nullptr};
  double* hist = nullptr;
  // resident grid loop (allocated by its first solve): tagged sum slots,
  // published boundary rows (tagged words), the failure flag, the time of the last
  // launch
  uint64_t* grid_slot = nullptr;
  uint64_t* grid_halo = nullptr;
  int* grid_fail = nullptr;
  int64_t grid_slot_words = 0;
  int64_t grid_halo_len = 0;
  hipEvent_t grid_ev[2] = {nullptr, nullptr};
  bool grid_timed = false;     // grid_ev hold the last launch
  // Jacobi workspace (allocated by the first preconditioned solve)
  double* jz = nullptr;
  double* jdiag = nullptr;
  int* jbad = nullptr;
  int64_t hist_cap = 0;
  int64_t hist_batch = 0;

  // graphs of `graph_block` iterations, keyed by batch size
  int64_t graph_block = 32;
  // solver workgroups per compute unit: 1, 2, or 0 (by problem size)
  int32_t wg_per_cu = 0;
  // SLA_ONE_GROUP_AUTO: systems of up to 2048 unknowns (banded, or tiles of
  // at most kWaveCap slots) run the CG loop in one workgroup per system, and
  // single banded systems that fit the chip in one cooperative launch (the
  // resident grid loop); SLA_ONE_GROUP_OFF: always the two-kernel loop
  int32_t one_group = SLA_ONE_GROUP_AUTO;
  // grid line length L of a band whose far offsets are +-L and whose other
  // offsets lie within +-63 (0: the line walk does not apply)
  int64_t line = 0;
  hipStream_t capture_stream = nullptr;
  // Lanczos basis and scratch, allocated by the first eigsh call
  sla::EigWork* eig = nullptr;
  // BiCGStab vectors, partials and scalars, allocated by the first solve
  sla::BsWork* bs = nullptr;
  bool bs_hist_valid = false;
  // sla_csr_reorder: CG solves and adjoints run on P A P^T (its own handle)
  sla::Reorder* ro = nullptr;
  std::map<int64_t, std::pair<hipGraph_t, hipGraphExec_t>> graphs;
};

namespace sla {

// Where a CG solve keeps its device state (r, both search directions, q, the
// partials, the context with the systems' scalar records, the running
// count) and the host copies it reads back: the handle's own workspace
// (own = true: captured graphs, history and Jacobi preconditioning allowed),
// or caller-provided memory such as the allocation-free entry point's static
// scratch (own = false: kernels launched one by one, no events).
struct CgSpace {
  double* r = nullptr;
  double* p0 = nullptr;
  double* p1 = nullptr;
  double* q = nullptr;
  double* part = nullptr;        // kPartSets * batch * grid
  Ctx* ctx_dev = nullptr;        // the context, then the batch's Scal records
  int* n_running = nullptr;
  Ctx* ctx_host = nullptr;       // host copy of the context
  Scal* scal_host = nullptr;     // [batch] host copies of the records
  int* poll_host = nullptr;      // [2]
  hipEvent_t* poll_ev = nullptr; // [2], or nullptr: wait for the stream at each poll
  int32_t grid = 0;              // solver workgroups per system
  bool own = true;
};

// The adjoint's tail on the one-workgroup loop: `gate` (a device int the
// values' symmetry check sets) stops the solve and the pattern gradient on
// the device, so no host round trip precedes the solve; grad_vals (or
// nullptr) receives -lambda_i x_j, enqueued before the solve's results are
// read back.
// Internal solve flag (never accepted from callers): keep the solve off the
// resident grid loop.  The list calls set it: their systems run concurrently
// on worker streams, which cooperative launches, each holding every CU,
// would serialize.
constexpr uint32_t kFlagNoResident = 0x40000000u;

struct AdjointTail {
  const int* gate = nullptr;
  const double* x = nullptr;
  double* grad_vals = nullptr;
};

// Workspace and launch helpers implemented in cg.hip
sla_status ensure_workspace(sla_csr A, int64_t batch);
// the solver grid (workgroups per system) of a solve of `batch` systems
int32_t solver_grid(const sla_csr A, int64_t batch);
// the CG loop of run_cg on a given space (flags: X0 always; HISTORY and
// JACOBI only on the handle's own space)
sla_status run_cg_space(sla_csr A, const CgSpace& sp, const double* b, double* x, double tol,
                        int64_t maxit, uint32_t flags, sla_cg_info* info, hipStream_t stream,
                        const AdjointTail* tail = nullptr);
bool use_band(const sla_csr A);   // banded SpMV kernels for this handle?
bool use_split(const sla_csr A);  // separate direction pass before the SpMV?
bool use_lines(const sla_csr A);  // line-walk SpMV step (a banded pattern with far offsets +-L)?
bool use_one_group(const sla_csr A);  // the one-workgroup-per-system CG loop?
// the resident grid loop for `batch` systems (with or without Jacobi)?
bool use_grid(const sla_csr A, int64_t batch, bool jacobi);
// duration of the last resident grid loop (SLA_ERR_ARG: none)
sla_status grid_loop_ms(sla_csr A, double* ms);
// y[s] = A_s^T x[s] (builds the transposed pattern on first use)
sla_status launch_spmv_transpose(sla_csr A, const double* x, double* y, hipStream_t st);
// grad_vals[s][k] = sign * g[s][i] * x[s][col[k]] on every stored slot;
// nothing is written when `gate` (a device int, or nullptr) is set
sla_status launch_slot_products(sla_csr A, int64_t batch, const double* g, const double* x,
                                double* out, bool negate, hipStream_t st,
                                const int* gate = nullptr);
void release_workspace(sla_csr A);
void free_handle(sla_csr A);  // the handle, its workspace and its transposed pattern
sla_status analyse_pattern(sla_csr A, hipStream_t stream);
// Symmetry of the pattern and, with values = true, of the bound values of
// every system (mirror entries equal to within 1e-12 relative): *bad gets
// bit 0 for a stored (i, j) whose mirror (j, i) is not stored, bit 1 for a
// mirror pair with different values.  flag_dev: a device int to use for the
// result (nullptr: the handle's own, allocated on first use).  Synchronises
// `stream` (csr_build.hip).
sla_status check_symmetry(sla_csr A, bool values, int* bad, hipStream_t stream,
                          int* flag_dev = nullptr);
// The same check enqueued only: *flag_out (device, the handle's flag) holds
// its result once the stream reaches it; nullptr for a pattern without slots.
sla_status enqueue_symmetry_check(sla_csr A, bool values, hipStream_t stream, int** flag_out);

sla_status launch_spmv(sla_csr A, const double* vals, int64_t batch, const double* x,
                       double* y, hipStream_t stream);
// y = A x plus per-workgroup partials of wdot.y (nd = 1) and of y.y (nd = 2)
// in part[system * pstride + set * groups + workgroup], groups =
// spmv_groups(A, batch)
sla_status launch_spmv_dots(sla_csr A, const double* vals, int64_t batch, const double* x,
                            double* y, const double* wdot, int nd, double* part, int64_t pstride,
                            int set0, int set1, hipStream_t stream);
int64_t spmv_groups(const sla_csr A, int64_t batch);
sla_status launch_pattern_grad(sla_csr A, int64_t batch, const double* lambda,
                               const double* x, double* grad_vals, hipStream_t stream);
sla_status run_cg(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                  uint32_t flags, sla_cg_info* info, hipStream_t stream,
                  const AdjointTail* tail = nullptr);
// Lanczos eigenpairs of every bound system (lanczos.hip)
sla_status run_eigsh(sla_csr A, int64_t k, int which, int64_t m, const double* v0,
                     double* theta, double* X, double* resid, sla_eig_info* info,
                     hipStream_t stream);
// grad[s][slot (i, j)] = sum_t g[s][t] X[s][t][i] X[s][t][j]
sla_status launch_eig_grad(sla_csr A, int64_t k, const double* X, const double* g,
                           double* grad, hipStream_t stream);
void release_eig_work(sla_csr A);
// BiCGStab (bicgstab.hip)
sla_status run_bicgstab(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                        uint32_t flags, sla_cg_info* info, hipStream_t stream);
sla_status run_bicgstab_adjoint(sla_csr A, const double* x, const double* grad_x,
                                double* grad_b, double* grad_vals, double tol, int64_t maxit,
                                uint32_t flags, sla_cg_info* info, hipStream_t stream);
sla_status bicgstab_history(sla_csr A, int64_t system, double* rho, double* alpha,
                            double* omega, double* rr, int64_t cap, int64_t* count);
void release_bs_work(sla_csr A);
// mean durations of the Gram-Schmidt dot and update passes over nvec basis
// vectors, on the basis an earlier eigsh left in the workspace
sla_status profile_lanczos_kernels(sla_csr A, int64_t nvec, int64_t reps, double* avg_ms,
                                   hipStream_t stream);
sla_status profile_kernels(sla_csr A, const double* b, double* x, int64_t reps,
                           double* avg_ms, hipStream_t stream);

// Locality ordering (reorder.hip): A->ro with the breadth-first order of the
// pattern's graph and the handle of P A P^T
sla_status make_reorder(sla_csr A, hipStream_t stream);
void release_reorder(sla_csr A);
// CG on A, or on P A P^T with b, x permuted in and out when A is reordered
sla_status run_cg_any(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                      uint32_t flags, sla_cg_info* info, hipStream_t stream);
// BiCGStab on A, or on P A P^T (the adjoint on its transpose, P A^T P^T)
sla_status run_bicgstab_any(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                            uint32_t flags, sla_cg_info* info, hipStream_t stream);
sla_status run_bicgstab_adjoint_any(sla_csr A, const double* x, const double* grad_x,
                                    double* grad_b, double* grad_vals, double tol,
                                    int64_t maxit, uint32_t flags, sla_cg_info* info,
                                    hipStream_t stream);
sla_status profile_kernels_any(sla_csr A, const double* b, double* x, int64_t reps,
                               double* avg_ms, hipStream_t stream);
sla_status copy_order(sla_csr A, int32_t* out, hipStream_t stream);
// the handle whose kernels and CG state a solve on A uses
sla_csr solver_handle(sla_csr A);

// COO / CSR construction implemented in csr_build.hip
sla_status build_from_coo(sla_csr A, sla_index coo_idx, const void* row,
                          const void* col, hipStream_t stream);
sla_status build_from_csr(sla_csr A, const void* rowptr, const int32_t* col,
                          hipStream_t stream);
// the transposed pattern A->trans (built once; csr_build.hip)
sla_status build_transpose(sla_csr A, hipStream_t stream);
sla_status launch_values_from_coo(sla_csr A, const double* coo_val, double* vals,
                                  int64_t batch, hipStream_t stream);
sla_status launch_grad_to_coo(sla_csr A, const double* grad_vals, double* grad_coo,
                              int64_t batch, hipStream_t stream);

}  // namespace sla
