#!/usr/bin/env python3
"""Benchmark of the CSR CG solve + adjoint on one MI355X.

One step is the whole hot path on the 1000 x 1000 Poisson workload
(n = 1e6, nnz = 4,996,000, int32 CSR, fp64): b = A u* with
u* = sin(pi x) sin(pi y), a forward CG solve of exactly 1000 iterations
(tol 0), then the adjoint solve of exactly 1000 iterations for
grad_x ~ N(0,1) (seed 1) and the pattern gradient -lambda_i x_j.  Inputs are
resident in HBM before timing starts.

Printed: ONE JSON line.  ``value`` is CG iterations per second over the
timed steps (forward + adjoint).  Extra fields: effective bandwidth on the
canonical bytes of one iteration (12 nnz + 4 (n+1) + 88 n; the 1M working
set is Infinity-Cache resident, so this is an effective rate), the roofline
of the dominant kernel (the resident grid CG loop, one launch per solve,
timed by the library's events around each launch), the library's own device
memory, and ``sizes``: the
same solve at 16M and 169M unknowns (500 fixed iterations, median of 3, each
with its roofline on canonical bytes and on the bytes the committed counters
saw, and the oracle's CG on the same system on all host threads: its time
and x's relative difference), the random geometric graph, the 64-system
batch and the 32 x 32 workload (each with an oracle leg), and the CPU oracle
on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--sizes 16m,169m]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "CG solve ms & iterations/s at 1M/16M/169M DOF fp64; effective HBM GB/s vs peak"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def canonical_bytes(n: int, nnz: int, rp_bytes: int) -> int:
    """Bytes one textbook CG iteration must move (matrix once; SpMV + p.Ap,
    axpy + r.r and the direction update each touching their vectors once)."""
    return 12 * nnz + rp_bytes * (n + 1) + 88 * n


def spmv_step_bytes(n: int, nnz: int, rp_bytes: int) -> int:
    """Algorithmic bytes of one launch of the fused SpMV step: the matrix
    (values, columns, row pointers) once, reads of r, p_{k-1}, x and writes of
    p_k, q, x."""
    return 12 * nnz + rp_bytes * (n + 1) + 48 * n


def spmv_step_bytes_banded(n: int, nnz: int, rp_bytes: int) -> int:
    """The same launch with the banded kernels: values once, one mask byte
    per row and one row pointer per 64-row tile instead of the column array
    and per-row row pointers."""
    tiles = (n + 63) // 64
    return 8 * nnz + n + rp_bytes * (tiles + 1) + 48 * n


def spmv_step_bytes_lines(n: int, nnz: int, rp_bytes: int) -> int:
    """The same launch with the line walk, averaged over two steps: x and the
    previous-but-one direction are read, and x written, at every other step
    only (read 32 n / 16 n, write 24 n / 16 n of vectors)."""
    tiles = (n + 63) // 64
    return 8 * nnz + n + rp_bytes * (tiles + 1) + 44 * n


def spmv_step_bytes_split(n: int, nnz: int, rp_bytes: int) -> int:
    """The SpMV step as two launches for wide-column patterns: the direction
    pass reads r, p_{k-1}, x and writes p_k, x (40 n); the product pass reads
    the matrix once and p_k, and writes q."""
    return 40 * n + 12 * nnz + rp_bytes * (n + 1) + 16 * n


def spmv_variant(P) -> str:
    if P.split:
        return "split"
    if P.lines:
        return "lines"
    return "banded" if P.banded else "csr"


# kernel that runs the SpMV step under each variant
STEP_KERNEL = {"lines": "k_cg_spmv_lines", "banded": "k_cg_spmv", "csr": "k_cg_spmv",
               "split": "k_cg_direction+k_cg_product"}


def spmv_bytes_for(variant: str, n: int, nnz: int, rp_bytes: int) -> int:
    """Algorithmic bytes of one SpMV step under `variant` (the line walk:
    the banded kernel's arrays, with x's updates applied two steps at a time,
    as the mean over two steps)."""
    if variant == "lines":
        return spmv_step_bytes_lines(n, nnz, rp_bytes)
    if variant == "banded":
        return spmv_step_bytes_banded(n, nnz, rp_bytes)
    if variant == "split":
        return spmv_step_bytes_split(n, nnz, rp_bytes)
    return spmv_step_bytes(n, nnz, rp_bytes)


def pattern_grad_bytes(n: int, nnz: int, rp_bytes: int) -> int:
    return 12 * nnz + rp_bytes * (n + 1) + 16 * n


def code_digest(files) -> str:
    """sha256/16 of the kernel sources with comments and blank space removed:
    a profile summary stays valid across edits of the comments only."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "krylov_solvers_adjoint_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def source_digest() -> str:
    return code_digest(("cg.hip", "common.h"))


def lanczos_digest() -> str:
    return code_digest(("lanczos.hip", "common.h"))


def traffic_from_profile(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_d = re.search(r"source digest:\s*([0-9a-f]+)", text)
    m_t = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not m_d or not m_t or m_d.group(1) != digest:
        return None
    return float(m_t.group(1))


def counter_rows(path_name: str, digest: str) -> dict:
    """{(kernel, size): (bytes read, bytes written) per launch} from the table
    of a committed counter summary (scaled FETCH_SIZE / WRITE_SIZE, in MB),
    if it was taken on the current kernel source (else {})."""
    path = os.path.join(PROFILE_DIR, path_name)
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    m_d = re.search(r"source digest:\s*([0-9a-f]+)", text)
    if not m_d or m_d.group(1) != digest:
        return {}
    rows = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) < 7 or not cells[0].startswith("k_"):
            continue
        try:
            rd = float(cells[5].split()[0]) * 1e6
            wr = float(cells[6].split()[0]) * 1e6
        except (ValueError, IndexError):
            continue
        rows[(cells[0], cells[1])] = (rd, wr)
    return rows


ITERATION_COUNTERS = "k_cg_spmv_lines_poisson1000_counters.md"


CSR_ONLY = False  # --csr-only: force the plain CSR kernels


def gpu_setup(N: int, rp_dtype):
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    t0 = time.time()
    rowptr, col, vals = W.poisson_csr(N, rp_dtype)
    log(f"[bench] generated Poisson {N}x{N}: n={N*N} nnz={len(col)} in {time.time()-t0:.1f}s")
    free0 = torch.cuda.mem_get_info()[0]
    P = K.sla_csr_create_from_csr(torch.from_numpy(rowptr).to(dev), torch.from_numpy(col).to(dev))
    if CSR_ONLY:
        P.set_spmv_variant("csr")
    v = torch.from_numpy(vals).to(dev)
    del rowptr, col
    return P, v, vals, free0


def bench_headline(args):
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    N = 1000
    n = N * N
    torch.cuda.synchronize()
    lib0, _ = K.sla_memory_usage(reset_peak=True)
    P, v, vals_np, free0 = gpu_setup(N, np.int32)
    u, b_np = W.manufactured(N)
    g_np = W.normal_rhs(n, 1)
    b = torch.from_numpy(b_np).to(dev)
    g = torch.from_numpy(g_np).to(dev)
    nnz = P.nnz
    its = 1000

    def step():
        x, fi = K.sla_cg_solve(P, v, b, 0.0, its)
        gb, gv, ai = K.sla_cg_adjoint(P, v, x, g, 0.0, its)
        return x, gb, gv, fi, ai

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # events around each half of a step (forward solve, adjoint) as well
    halves = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    e0.record(stream)
    for ea, em, ez in halves:
        ea.record(stream)
        x, fi = K.sla_cg_solve(P, v, b, 0.0, its)
        em.record(stream)
        gb, gv, ai = K.sla_cg_adjoint(P, v, x, g, 0.0, its)
        ez.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    fwd_ms = sum(ea.elapsed_time(em) for ea, em, _ in halves) / args.steps
    adj_ms = sum(em.elapsed_time(ez) for _, em, ez in halves) / args.steps
    free1 = torch.cuda.mem_get_info()[0]
    lib1, libpeak = K.sla_memory_usage()
    total_iters = (fi.iterations + ai.iterations) * args.steps
    step_bytes = (fi.iterations + ai.iterations) * canonical_bytes(n, nnz, 4) + \
        pattern_grad_bytes(n, nnz, 4)
    ms_per_step = 1e3 * wall / args.steps
    # sanity: the manufactured solution is recovered
    err = float(torch.linalg.norm(x - torch.from_numpy(u).to(dev)) /
                torch.linalg.norm(torch.from_numpy(u).to(dev)))
    # the resident grid loop (the whole solve in one cooperative launch):
    # the library's events around each launch of a forward solve
    loop_ms = []
    for _ in range(max(3, args.steps)):
        K.sla_cg_solve(P, v, b, 0.0, its)
        try:
            loop_ms.append(K.sla_resident_loop_ms(P))
        except K.SlaError:
            break
    # the two-kernel loop's iteration kernels on the same handle, for comparison
    kern = K.sla_profile_iteration_kernels(P, v, b, reps=args.kernel_reps)
    # the pattern gradient on its own (grad_vals = -lambda_i x_j), event-timed
    pg_ms = _event_ms(lambda: K.sla_pattern_grad(P, v, gb, x), args.kernel_reps)
    pg_bytes = pattern_grad_bytes(n, nnz, 4)
    torch.cuda.synchronize()
    res = dict(
        n=n, nnz=nnz, iterations_fwd=fi.iterations, iterations_adj=ai.iterations,
        forward_ms=fwd_ms, adjoint_ms=adj_ms,
        pattern_grad=dict(ms=pg_ms, bytes=pg_bytes, GBps=pg_bytes / (pg_ms * 1e-3) / 1e9),
        ms_per_step=ms_per_step, gpu_ms_per_step=gpu_ms / args.steps,
        it_per_s=total_iters / wall,
        eff_GBps=step_bytes * args.steps / wall / 1e9,
        solution_rel_error=err,
        free_delta_MB=(free0 - free1) / 2**20,
        library_MB=(lib1 - lib0) / 1e6,
        library_peak_MB=(libpeak - lib0) / 1e6,
        # the caller's tensors of one forward + adjoint step: values, b, grad_x
        # (inputs), x, grad_b, grad_vals (outputs)
        caller_MB=(8 * nnz * 2 + 8 * n * 4) / 1e6,
        kernel_ms=kern,
    )
    res["pct_peak_effective"] = 100.0 * res["eff_GBps"] / HBM_PEAK_GBPS
    res["loop"] = "resident" if loop_ms else "two-kernel"
    res["loop_ms"] = sum(loop_ms) / len(loop_ms) if loop_ms else None
    res["loop_ms_runs"] = loop_ms
    res["loop_iterations"] = its
    res["spmv"] = spmv_variant(P)
    res["spmv_bytes"] = spmv_bytes_for(res["spmv"], n, nnz, 4)
    del P
    torch.cuda.synchronize()
    return res


def bench_head_solves(reps: int) -> dict:
    """The headline's forward solve (Poisson 1000^2, b = A u*, 1000 fixed
    iterations) `reps` times after one untimed: the resident loop's launch
    times (for the profiler passes on that launch)."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    P, v, _, _ = gpu_setup(1000, np.int32)
    _, b_np = W.manufactured(1000)
    b = torch.from_numpy(b_np).to(v.device)
    K.sla_cg_solve(P, v, b, 0.0, 1000)
    ms = []
    for _ in range(reps):
        K.sla_cg_solve(P, v, b, 0.0, 1000)
        ms.append(K.sla_resident_loop_ms(P))
    torch.cuda.synchronize()
    return dict(loop_ms=ms, iterations=1000)


def bench_size(N: int, rp_dtype, its: int, kernel_reps: int, runs: int = 5, warmups: int = 2):
    """Poisson N x N, b ~ U(-1,1) seed 0, `its` fixed CG iterations: the
    median of `runs` solves timed with HIP events on the solve's stream after
    `warmups` untimed ones, per-kernel times, the roofline of the SpMV step
    and of the whole iteration (canonical bytes and the bytes the committed
    counters saw), and the library's device memory.  Also returns (b, x) on
    the host for the oracle leg."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    n = N * N
    torch.cuda.synchronize()
    lib0, _ = K.sla_memory_usage(reset_peak=True)
    P, v, _, free0 = gpu_setup(N, rp_dtype)
    rp_bytes = 8 if rp_dtype == np.int64 else 4
    b_np = W.uniform_rhs(n, 0)
    b = torch.from_numpy(b_np).to(dev)
    # warm-ups: capture the iteration graph and touch the workspace
    for _ in range(warmups):
        K.sla_cg_solve(P, v, b, 0.0, its)
    torch.cuda.synchronize()
    walls = []
    stream = torch.cuda.current_stream()
    for _ in range(runs):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        x, info = K.sla_cg_solve(P, v, b, 0.0, its, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        walls.append(1e-3 * e0.elapsed_time(e1))
    wall = float(np.median(walls))
    free1 = torch.cuda.mem_get_info()[0]
    lib1, libpeak = K.sla_memory_usage()
    x_np = x.cpu().numpy()
    kern = K.sla_profile_iteration_kernels(P, v, b, reps=kernel_reps)
    nnz = P.nnz
    variant = spmv_variant(P)
    sbytes = spmv_bytes_for(variant, n, nnz, rp_bytes)
    cbytes = canonical_bytes(n, nnz, rp_bytes)
    ms_it = 1e3 * wall / info.iterations
    out = dict(n=n, nnz=nnz, rowptr="i64" if rp_bytes == 8 else "i32", spmv=variant,
               iterations=info.iterations, runs=runs,
               solve_ms=1e3 * wall, solve_ms_runs=[1e3 * w for w in walls],
               ms_per_iteration=ms_it,
               it_per_s=info.iterations / wall,
               canonical_bytes_per_iteration=cbytes,
               canonical_GBps=cbytes / (ms_it * 1e-3) / 1e9,
               rel_residual=info.rel_residual,
               free_delta_MB=(free0 - free1) / 2**20,
               library_MB=(lib1 - lib0) / 1e6,
               library_peak_MB=(libpeak - lib0) / 1e6,
               kernel_ms=kern,
               spmv_GBps=sbytes / (kern["spmv_step"] * 1e-3) / 1e9)
    out["pct_peak_canonical"] = 100.0 * out["canonical_GBps"] / HBM_PEAK_GBPS
    size = {1000: "1M", 4000: "16M", 13000: "169M"}.get(N)
    out["roofline"] = iteration_roofline(variant, n, nnz, rp_bytes, kern, ms_it, size)
    del P, v, b, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out, b_np, x_np


def iteration_roofline(variant: str, n: int, nnz: int, rp_bytes: int, kern: dict,
                       ms_it: float, size):
    """The SpMV step's roofline (its algorithmic bytes over its live event
    time, and the counters' bytes per launch when the committed summary was
    taken on the current source), and the whole iteration against peak on
    canonical bytes and on the bytes the counters saw per iteration."""
    kname = STEP_KERNEL[variant]
    sbytes = spmv_bytes_for(variant, n, nnz, rp_bytes)
    spmv_ms = kern["spmv_step"]
    achieved = sbytes / (spmv_ms * 1e-3) / 1e9
    rows = counter_rows(ITERATION_COUNTERS, source_digest()) if size else {}
    sp = rows.get((kname, size))
    rs = rows.get(("k_cg_residual", size))
    roof = dict(bound="hbm", kernel=kname, achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                frac=achieved / HBM_PEAK_GBPS, kernel_ms=spmv_ms, algorithmic_bytes=sbytes,
                traffic=(sp[0] + sp[1]) if sp else None, source_digest=source_digest())
    roof["frac_canonical"] = canonical_bytes(n, nnz, rp_bytes) / (ms_it * 1e-3) / 1e9 / \
        HBM_PEAK_GBPS
    if sp:
        roof["frac_kernel_moved"] = (sp[0] + sp[1]) / (spmv_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS
    if sp and rs:
        moved = sp[0] + sp[1] + rs[0] + rs[1]
        roof["moved_bytes_per_iteration"] = moved
        roof["frac_iteration_moved"] = moved / (ms_it * 1e-3) / 1e9 / HBM_PEAK_GBPS
        roof["residual_frac_moved"] = (rs[0] + rs[1]) / (kern["residual_step"] * 1e-3) / 1e9 / \
            HBM_PEAK_GBPS
    return roof


def bench_batch64(kernel_reps: int):
    """The shared-pattern batch: 64 Poisson 128 x 128 systems (diagonal
    4 + c_s), CG to tol 1e-8 forward and adjoint; iteration time while all
    64 are active, from the per-kernel timing launches."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    N, B = 128, 64
    rp, c, vals, b, _ = W.batched_poisson(N, B, 2, 3)
    g = W.normal_rhs(N * N, 4, shape=(B, N * N))
    P = K.sla_csr_create_from_csr(torch.from_numpy(rp).to(dev), torch.from_numpy(c).to(dev))
    vt = torch.from_numpy(vals).to(dev)
    bt = torch.from_numpy(b).to(dev)
    gt = torch.from_numpy(g).to(dev)
    K.sla_cg_solve_batched(P, vt, bt, 1e-8, 50)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    x, fi = K.sla_cg_solve_batched(P, vt, bt, 1e-8, 10000)
    gb, gv, ai = K.sla_cg_adjoint_batched(P, vt, x, gt, 1e-8, 10000)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n, nnz = N * N, P.nnz
    its_f = [i.iterations for i in fi]
    its_a = [i.iterations for i in ai]
    # canonical bytes of one iteration of all 64 systems: the pattern read
    # once, the values and vectors per system
    b_it = B * (8 * nnz + 88 * n) + 4 * nnz + 4 * (n + 1)
    out = dict(systems=B, n=n, nnz=nnz, iterations_fwd=[min(its_f), max(its_f)],
               iterations_adj=[min(its_a), max(its_a)], solve_adjoint_ms=1e3 * wall,
               steps=max(its_f) + max(its_a),
               us_per_step=1e6 * wall / (max(its_f) + max(its_a)),
               canonical_bytes_all_active=b_it,
               eff_GBps_upper=b_it * (max(its_f) + max(its_a)) / wall / 1e9)
    del P, vt, bt, gt, x, gb, gv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def bench_poisson32():
    """The 32 x 32 Poisson workload (tol 1e-10, forward + adjoint; b ~ U(-1,1)
    seed 0, g ~ N(0,1) seed 1) and a batch of 256 shifted 32 x 32 systems,
    each through the one-workgroup CG loop (the default at this size) and the
    two-kernel loop; median of 20 timed calls."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    rp, c, v = W.poisson_csr(32)
    rpt, ct = torch.from_numpy(rp).to(dev), torch.from_numpy(c).to(dev)
    vt = torch.from_numpy(v).to(dev)
    bt = torch.from_numpy(W.uniform_rhs(1024, 0)).to(dev)
    gt = torch.from_numpy(W.normal_rhs(1024, 1)).to(dev)
    rpb, cb, vals_b, b_b, _ = W.batched_poisson(32, 256, 2, 3)
    vbt = torch.from_numpy(vals_b).to(dev)
    bbt = torch.from_numpy(b_b).to(dev)
    gbt = torch.from_numpy(W.normal_rhs(1024, 4, shape=(256, 1024))).to(dev)
    out = {}
    for mode, key in (("auto", "one_group"), ("off", "two_kernel")):
        P = K.sla_csr_create_from_csr(rpt, ct)
        P.set_one_group(mode)
        times, ftimes, btimes = [], [], []
        for rep in range(22):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            x, fi = K.sla_cg_solve(P, vt, bt, 1e-10, 10000)  # returns after the solve
            tm = time.perf_counter()
            gb, gv, ai = K.sla_cg_adjoint(P, vt, x, gt, 1e-10, 10000)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            ftimes.append(tm - t0)
            t0 = time.perf_counter()
            xb, fb = K.sla_cg_solve_batched(P, vbt, bbt, 1e-10, 10000)
            gbb, gvb, ab = K.sla_cg_adjoint_batched(P, vbt, xb, gbt, 1e-10, 10000)
            torch.cuda.synchronize()
            btimes.append(time.perf_counter() - t0)
        ms = 1e3 * float(np.median(times[2:]))
        bms = 1e3 * float(np.median(btimes[2:]))
        its = fi.iterations + ai.iterations
        steps = max(i.iterations for i in fb) + max(i.iterations for i in ab)
        out[key] = dict(iterations_fwd=fi.iterations, iterations_adj=ai.iterations,
                        solve_adjoint_ms=ms, us_per_iteration=1e3 * ms / its,
                        forward_ms=1e3 * float(np.median(ftimes[2:])),
                        adjoint_ms=1e3 * float(np.median(np.subtract(times, ftimes)[2:])),
                        batch256_ms=bms, batch256_us_per_step=1e3 * bms / steps)
        del P
    out["speedup"] = out["two_kernel"]["solve_adjoint_ms"] / out["one_group"]["solve_adjoint_ms"]
    out["batch256_speedup"] = out["two_kernel"]["batch256_ms"] / out["one_group"]["batch256_ms"]
    torch.cuda.synchronize()
    return out


def bench_rgg(n: int, kernel_reps: int):
    """Random geometric graph Laplacian + 0.01 I (4M nodes, ~9 slots per row,
    random node order): CSR built on the GPU from COO, then CG to 1e-8 and the
    adjoint to 1e-8."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    t0 = time.time()
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    b = torch.from_numpy(W.normal_rhs(n, 6)).to(dev)
    g = torch.from_numpy(W.normal_rhs(n, 7)).to(dev)
    log(f"[bench] generated RGG n={n} triplets={row.shape[0]} in {time.time()-t0:.1f}s")
    rt = torch.from_numpy(row.astype(np.int32)).to(dev)
    ct = torch.from_numpy(col.astype(np.int32)).to(dev)
    vt = torch.from_numpy(val).to(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    P = K.sla_csr_create(n, rt, ct)
    v = K.sla_csr_values_from_coo(P, vt)
    torch.cuda.synchronize()
    build_ms = 1e3 * (time.perf_counter() - t0)
    if CSR_ONLY:
        P.set_spmv_variant("csr")
    K.sla_cg_solve(P, v, b, 1e-8, 50)  # warm-up (graph capture)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    x, fi = K.sla_cg_solve(P, v, b, 1e-8, 20000)
    torch.cuda.synchronize()
    fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    gb, gv, ai = K.sla_cg_adjoint(P, v, x, g, 1e-8, 20000)
    torch.cuda.synchronize()
    adj = time.perf_counter() - t0
    # the same solve and adjoint preconditioned with diag(A) (the pages' Jacobi)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    xj, fj = K.sla_cg_solve(P, v, b, 1e-8, 20000, jacobi=True)
    gbj, gvj, aj = K.sla_cg_adjoint(P, v, xj, g, 1e-8, 20000, jacobi=True)
    torch.cuda.synchronize()
    jac_s = time.perf_counter() - t0
    jacobi = dict(iterations_fwd=fj.iterations, iterations_adj=aj.iterations,
                  solve_adjoint_ms=1e3 * jac_s,
                  it_per_s=(fj.iterations + aj.iterations) / jac_s)
    del xj, gbj, gvj
    kern = K.sla_profile_iteration_kernels(P, v, b, reps=kernel_reps)
    nnz = P.nnz
    its = fi.iterations + ai.iterations
    sbytes = spmv_bytes_for(spmv_variant(P), n, nnz, 4)
    out = dict(n=n, nnz=nnz, spmv=spmv_variant(P), csr_build_ms=build_ms,
               iterations_fwd=fi.iterations, iterations_adj=ai.iterations,
               solve_ms=1e3 * fwd, adjoint_ms=1e3 * adj,
               it_per_s=its / (fwd + adj),
               eff_GBps=(its * canonical_bytes(n, nnz, 4) + pattern_grad_bytes(n, nnz, 4)) /
               (fwd + adj) / 1e9,
               kernel_ms=kern,
               spmv_GBps=sbytes / (kern["spmv_step"] * 1e-3) / 1e9,
               jacobi=jacobi)
    out["pct_peak_canonical"] = 100.0 * out["eff_GBps"] / HBM_PEAK_GBPS
    # the same solve and adjoint after renumbering the unknowns in the
    # breadth-first order of the graph (sla_csr_reorder): the time per call
    # includes gathering the values and permuting b / x in and out
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    P.reorder()
    torch.cuda.synchronize()
    order_ms = 1e3 * (time.perf_counter() - t0)
    K.sla_cg_solve(P, v, b, 1e-8, 50)  # warm-up (graph capture on the permuted copy)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    xr, ri = K.sla_cg_solve(P, v, b, 1e-8, 20000)
    gbr, gvr, rai = K.sla_cg_adjoint(P, v, xr, g, 1e-8, 20000)
    torch.cuda.synchronize()
    rs = time.perf_counter() - t0
    rkern = K.sla_profile_iteration_kernels(P, v, b, reps=kernel_reps)
    rits = ri.iterations + rai.iterations
    # Jacobi preconditioning on the reordered copy
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    xrj, rj = K.sla_cg_solve(P, v, b, 1e-8, 20000, jacobi=True)
    gbrj, gvrj, raj = K.sla_cg_adjoint(P, v, xrj, g, 1e-8, 20000, jacobi=True)
    torch.cuda.synchronize()
    rjs = time.perf_counter() - t0
    del xrj, gbrj, gvrj
    out["reordered"] = dict(
        order_ms=order_ms, spmv=spmv_variant(P), iterations_fwd=ri.iterations,
        iterations_adj=rai.iterations, solve_adjoint_ms=1e3 * rs, it_per_s=rits / rs,
        eff_GBps=(rits * canonical_bytes(n, nnz, 4) + pattern_grad_bytes(n, nnz, 4)) / rs / 1e9,
        kernel_ms=rkern,
        spmv_GBps=spmv_bytes_for(spmv_variant(P), n, nnz, 4) / (rkern["spmv_step"] * 1e-3) / 1e9,
        jacobi=dict(iterations_fwd=rj.iterations, iterations_adj=raj.iterations,
                    solve_adjoint_ms=1e3 * rjs,
                    it_per_s=(rj.iterations + raj.iterations) / rjs))
    out["reordered"]["pct_peak_canonical"] = 100.0 * out["reordered"]["eff_GBps"] / HBM_PEAK_GBPS
    del P, v, b, g, x, gb, gv, xr, gbr, gvr
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def spmv_bytes(variant: str, n: int, nnz: int, rp_bytes: int) -> int:
    """Algorithmic bytes of y = A x: the matrix once (banded: values, a mask
    byte per row, a row pointer per 64 rows; else values, columns, row
    pointers), x read once, y written once."""
    if variant in ("lines", "banded"):
        return 8 * nnz + n + rp_bytes * ((n + 63) // 64 + 1) + 16 * n
    return 12 * nnz + rp_bytes * (n + 1) + 16 * n


def _event_ms(fn, reps: int) -> float:
    import torch
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_matvec(reps: int, N: int = 1000):
    """The differentiable .matvec on the N x N Poisson matrix: y = A x,
    y = A^T x (values gathered into the transposed pattern's order on each
    call) and the backward pass (grad_x = A^T g plus grad_vals = g_i x_j).
    At N = 1000 the matrix and vectors fit the Infinity Cache; at N = 4000
    they come from HBM."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    n = N * N
    P, v, _, _ = gpu_setup(N, np.int32)
    x = torch.from_numpy(W.normal_rhs(n, 2)).to(dev)
    g = torch.from_numpy(W.normal_rhs(n, 3)).to(dev)
    nnz = P.nnz
    variant = "banded" if P.banded else "csr"
    fwd = _event_ms(lambda: K.sla_spmv(P, v, x), reps)
    trn = _event_ms(lambda: K.sla_spmv_transpose(P, v, x), reps)
    bwd = _event_ms(lambda: K.sla_matvec_grad(P, v, x, g), reps)
    b_fwd = spmv_bytes(variant, n, nnz, 4)
    # A^T x through the transposed pattern: its columns and its map to A's
    # slots (4 B each per slot), A's values (8 B per slot), its row pointers,
    # x read and y written once
    b_trn = 16 * nnz + 4 * (n + 1) + 16 * n
    # plus grad_vals = g_i x_j: row pointers, columns, g and x read, 8 B
    # written per slot
    b_bwd = b_trn + 12 * nnz + 4 * (n + 1) + 16 * n
    out = dict(n=n, nnz=nnz, spmv=variant,
               spmv_ms=fwd, spmv_GBps=b_fwd / (fwd * 1e-3) / 1e9,
               transpose_ms=trn, transpose_GBps=b_trn / (trn * 1e-3) / 1e9,
               backward_ms=bwd, backward_GBps=b_bwd / (bwd * 1e-3) / 1e9,
               bytes=dict(spmv=b_fwd, transpose=b_trn, backward=b_bwd))
    del P, v, x, g
    torch.cuda.synchronize()
    return out


def lanczos_bytes(n: int, steps: int, k: int, spmv: int) -> int:
    """Algorithmic bytes of `steps` Lanczos steps with two Gram-Schmidt passes
    (step j reads the j + 1 basis vectors four times: two dot passes, two
    updates; w is read 4 times and written twice, v_{j+1} read and written
    once) plus the start and the k Ritz vectors."""
    gs = 8 * n * (2 * steps * (steps + 1) + 8 * steps)
    return gs + steps * spmv + 24 * n + 8 * n * (steps + k)


def bench_eigsh(m: int, k: int, N: int = 1000):
    """The .eigsh on the N x N Poisson matrix: the k largest eigenvalues by m
    Lanczos steps with full reorthogonalisation."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    n = N * N
    P, v, _, free0 = gpu_setup(N, np.int32)
    v0 = torch.from_numpy(W.normal_rhs(n, 72)).to(dev)
    K.sla_eigsh(P, v, k, "LA", m, v0)  # workspace, warm caches
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    t0 = time.perf_counter()
    th, X, res, infos = K.sla_eigsh(P, v, k, "LA", m, v0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps = infos[0].steps
    nbytes = lanczos_bytes(n, steps, k, spmv_bytes("banded" if P.banded else "csr", n, P.nnz, 4))
    grad_ms = _event_ms(lambda: K.sla_eig_grad(P, v, X, torch.ones(k, dtype=torch.float64,
                                                                   device=dev)), 10)
    # the Gram-Schmidt passes at the mean basis size of the run (step j
    # passes over j + 1 vectors): timed live with HIP events on the stream
    # they run on
    nvec = max(1, (steps + 1) // 2)
    gs = K.sla_profile_lanczos_kernels(P, nvec, reps=10)
    dot_bytes = 8 * n * (nvec + 1)        # nvec basis vectors and w read once
    upd_bytes = 8 * n * (nvec + 2)        # nvec basis vectors and w read, w written
    gs_roof = dict(nvec=nvec, dot_ms=gs["dot"], update_ms=gs["update"],
                   dot_GBps=dot_bytes / (gs["dot"] * 1e-3) / 1e9,
                   update_GBps=upd_bytes / (gs["update"] * 1e-3) / 1e9,
                   dot_bytes=dot_bytes, update_bytes=upd_bytes)
    out = dict(n=n, nnz=P.nnz, k=k, m=m, steps=steps, ms=1e3 * wall,
               steps_per_s=steps / wall, eff_GBps=nbytes / wall / 1e9,
               algorithmic_bytes=nbytes, basis_MB=(free0 - free1) / 2**20,
               theta=th.cpu().tolist(), resid=res.cpu().tolist(),
               # largest eigenvalue of the 5-point Laplacian, 4 + 4 cos(pi / (N + 1))
               theta_top_exact=4.0 + 4.0 * float(np.cos(np.pi / (N + 1))),
               eig_grad_ms=grad_ms)
    out["roofline"] = dict(
        bound="hbm", kernel="k_lz_dot (Gram-Schmidt dot pass)",
        achieved=gs_roof["dot_GBps"], peak=HBM_PEAK_GBPS, unit="GB/s",
        frac=gs_roof["dot_GBps"] / HBM_PEAK_GBPS,
        traffic=(traffic_from_profile("k_lz_dot", "poisson1000_m300", lanczos_digest())
                 if (N, m) == (1000, 300) else None),
        **{k_: v_ for k_, v_ in gs_roof.items()})
    del P, v, v0, th, X, res
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def bicgstab_bytes(n: int, nnz: int, variant: str) -> int:
    """Algorithmic bytes of one BiCGStab iteration: two SpMVs (A p, A s),
    which also read rhat and s for their dot products, and the vector passes:
    p = r + beta (p - omega v) reads r, p, v and writes p; s = r - alpha v
    reads 2, writes 1; the update reads s, x, p, t, rhat and writes x, r
    (16 vectors in all besides the SpMVs' own)."""
    return 2 * spmv_bytes(variant, n, nnz, 4) + 16 * 8 * n


def bench_bicgstab(N: int = 1000, fixed: int = 0):
    """BiCGStab forward + adjoint on the N x N upwind convection-diffusion
    matrix (non-symmetric) to tol 1e-8, or `fixed` iterations each (tol 0)."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    n = N * N
    tol, maxit = (0.0, fixed) if fixed else (1e-8, 10000)
    rp, c, v = W.convection_diffusion_csr(N)
    P = K.sla_csr_create_from_csr(torch.from_numpy(rp).to(dev), torch.from_numpy(c).to(dev))
    vt = torch.from_numpy(v).to(dev)
    b = torch.from_numpy(W.normal_rhs(n, 90)).to(dev)
    g = torch.from_numpy(W.normal_rhs(n, 91)).to(dev)
    K.sla_bicgstab_solve(P, vt, b, 1e-8, 40)  # workspace, transposed pattern below
    K.sla_bicgstab_adjoint(P, vt, b, g, 1e-8, 40)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    x, fi = K.sla_bicgstab_solve(P, vt, b, tol, maxit)
    torch.cuda.synchronize()
    fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    gb, gv, ai = K.sla_bicgstab_adjoint(P, vt, x, g, tol, maxit)
    torch.cuda.synchronize()
    adj = time.perf_counter() - t0
    variant = "banded" if P.banded else "csr"
    its = fi[0].iterations + ai[0].iterations
    nb = its * bicgstab_bytes(n, P.nnz, variant)
    bpi = bicgstab_bytes(n, P.nnz, variant)
    achieved = bpi / ((fwd + adj) / its) / 1e9
    out = dict(n=n, nnz=P.nnz, spmv=variant, iterations_fwd=fi[0].iterations,
               iterations_adj=ai[0].iterations, solve_ms=1e3 * fwd, adjoint_ms=1e3 * adj,
               roofline=dict(bound="hbm", kernel="the whole iteration (2 SpMVs with fused dot "
                             "partials + 3 vector kernels, graph-replayed)",
                             achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBPS, traffic=None,
                             algorithmic_bytes=bpi),
               it_per_s=its / (fwd + adj), us_per_iteration=1e6 * (fwd + adj) / its,
               eff_GBps=nb / (fwd + adj) / 1e9, bytes_per_iteration=bicgstab_bytes(n, P.nnz,
                                                                                    variant),
               rel_residual=fi[0].rel_residual)
    del P, vt, b, g, x, gb, gv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def bench_list(count: int = 32):
    """SparseTensorList: `count` Poisson systems with distinct grids (N = 100,
    110, ..., 410: distinct patterns and sizes), CG to tol 1e-8, solved as one
    list call (up to 8 at once) and one after another."""
    import numpy as np
    import torch
    import krylov_solvers_adjoint_amd as K
    import workloads as W
    dev = torch.device("cuda", 0)
    Ps, vals, bs = [], [], []
    for i in range(count):
        N = 100 + 10 * i
        rp, c, v = W.poisson_csr(N)
        Ps.append(K.sla_csr_create_from_csr(torch.from_numpy(rp).to(dev),
                                            torch.from_numpy(c).to(dev)))
        vals.append(torch.from_numpy(v).to(dev))
        bs.append(torch.from_numpy(W.uniform_rhs(N * N, i)).to(dev))
    K.sla_solve_list(Ps, vals, bs, 1e-8, 20000)  # workspaces, graphs
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    xs, infos = K.sla_solve_list(Ps, vals, bs, 1e-8, 20000)
    torch.cuda.synchronize()
    t_list = time.perf_counter() - t0
    t0 = time.perf_counter()
    for P, v, b in zip(Ps, vals, bs):
        K.sla_cg_solve(P, v, b, 1e-8, 20000)
    torch.cuda.synchronize()
    t_seq = time.perf_counter() - t0
    its = sum(i.iterations for i in infos)
    out = dict(systems=count, unknowns=int(sum(P.n for P in Ps)), iterations=its,
               list_ms=1e3 * t_list, sequential_ms=1e3 * t_seq,
               systems_per_s=count / t_list, speedup=t_seq / t_list,
               all_converged=all(i.converged for i in infos))
    del Ps, vals, bs, xs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _oracle_threads(threads: int | None = None):
    """Set the oracle's OpenMP threads: `threads`, or the process's CPU share
    (OMP_NUM_THREADS where the environment fixes it, else the CPUs this
    process may use)."""
    import oracle
    oracle.set_threads(threads if threads else oracle.host_threads())
    return oracle.get_threads()


def _cpu_fields(cores: int) -> dict:
    import oracle
    return dict(cores=cores, cpu_model=oracle.cpu_model(), cpus_visible=os.cpu_count(),
                kind="oracle")


def oracle_fixed(N: int, rp_dtype, b_np, x_gpu, its: int = 500) -> dict:
    """The oracle's CG on the same Poisson system, all `its` iterations on the
    process's host threads: the time, and x against the GPU's (parity)."""
    import numpy as np
    import oracle
    import workloads as W
    cores = _oracle_threads()
    rp, c, v = W.poisson_csr(N, np.int64)
    A = oracle.CSR(N * N, rp, c, v)
    t0 = time.perf_counter()
    xo, io = oracle.cg(A, b_np, 0.0, its)
    dt = time.perf_counter() - t0
    rel = float(np.linalg.norm(x_gpu - xo) / np.linalg.norm(xo))
    return dict(cpu_ms=1e3 * dt, cpu_it_per_s=io.iterations / dt, **_cpu_fields(cores),
                sample=f"all {io.iterations} iterations (the same solve)",
                oracle_iterations=io.iterations, oracle_rel_x=rel)


def oracle_one_thread_poisson(N: int, its: int) -> dict:
    """The oracle's CG on one thread on a bounded sample: `its` iterations of
    the N x N Poisson system (b ~ U(-1,1) seed 0)."""
    import numpy as np
    import oracle
    import workloads as W
    _oracle_threads(1)
    rp, c, v = W.poisson_csr(N, np.int64)
    A = oracle.CSR(N * N, rp, c, v)
    t0 = time.perf_counter()
    oracle.cg(A, W.uniform_rhs(N * N, 0), 0.0, its)
    dt = time.perf_counter() - t0
    out = dict(cpu_it_per_s=its / dt, **_cpu_fields(1),
               sample=f"{its} iterations on one thread, {dt:.1f} s")
    _oracle_threads()
    return out


def oracle_poisson32() -> dict:
    """The 32 x 32 workload on the oracle, one thread: tol 1e-10 forward +
    adjoint, the whole solve (a fraction of a second)."""
    import numpy as np
    import oracle
    import workloads as W
    _oracle_threads(1)
    rp, c, v = W.poisson_csr(32, np.int64)
    A = oracle.CSR(1024, rp, c, v)
    b, g = W.uniform_rhs(1024, 0), W.normal_rhs(1024, 1)
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        x, fi = oracle.cg(A, b, 1e-10, 10000)
        _, _, ai = oracle.adjoint(A, x, g, 1e-10, 10000)
    dt = (time.perf_counter() - t0) / reps
    _oracle_threads()
    return dict(cpu_ms=1e3 * dt, cpu_it_per_s=(fi.iterations + ai.iterations) / dt,
                **_cpu_fields(1), sample=f"the whole forward + adjoint ({fi.iterations} + "
                f"{ai.iterations} iterations), mean of {reps}")


def oracle_batch64() -> dict:
    """The 64-system batch on the oracle, one thread: every system's forward
    and adjoint solve to tol 1e-8, the whole workload."""
    import oracle
    import workloads as W
    _oracle_threads(1)
    N, B = 128, 64
    rp, c, vals, b, _ = W.batched_poisson(N, B, 2, 3)
    g = W.normal_rhs(N * N, 4, shape=(B, N * N))
    t0 = time.perf_counter()
    xs, infos = oracle.cg_batched(rp.astype("int64"), c, vals, b, 1e-8, 10000)
    _, _, ainfos = oracle.adjoint_batched(rp.astype("int64"), c, vals, xs, g, 1e-8, 10000)
    dt = time.perf_counter() - t0
    its = sum(i.iterations for i in infos) + sum(i.iterations for i in ainfos)
    _oracle_threads()
    return dict(cpu_ms=1e3 * dt, cpu_it_per_s=its / dt, **_cpu_fields(1),
                sample=f"the whole workload: {its} system-iterations")


def oracle_rgg(n: int, its: int = 60) -> dict:
    """The random geometric graph on the oracle, all host threads: its own
    CSR build from the same COO, then `its` CG iterations (a bounded sample
    of the tol 1e-8 forward + adjoint)."""
    import oracle
    import workloads as W
    cores = _oracle_threads()
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    t0 = time.perf_counter()
    rp, c, perm = oracle.csr_from_coo(n, row, col)
    vals = oracle.values_from_coo(perm, int(rp[-1]), val)
    build = time.perf_counter() - t0
    A = oracle.CSR(n, rp, c, vals)
    t0 = time.perf_counter()
    oracle.cg(A, W.normal_rhs(n, 6), 0.0, its)
    dt = time.perf_counter() - t0
    return dict(cpu_it_per_s=its / dt, csr_build_ms=1e3 * build, **_cpu_fields(cores),
                sample=f"the oracle's CSR build from the same COO ({build:.1f} s) and {its} "
                       f"CG iterations ({dt:.1f} s)")


def oracle_next(nxt: dict):
    """The oracle beside each NEXT leg, on bounded samples of the same
    workloads (a few seconds each), in the legs' own units."""
    import numpy as np
    import oracle
    import workloads as W
    cores = _oracle_threads()
    N = 1000
    n = N * N
    out = {}
    if "matvec" in nxt:
        rp, c, v = W.poisson_csr(N, np.int64)
        A = oracle.CSR(n, rp, c, v)
        x = W.normal_rhs(n, 2)
        t0 = time.perf_counter()
        for _ in range(100):
            oracle.spmv(A, x)
        fwd = (time.perf_counter() - t0) / 100
        t0 = time.perf_counter()
        for _ in range(20):
            oracle.matvec_grad(A, x, x)
        bwd = (time.perf_counter() - t0) / 20
        out["matvec"] = dict(spmv_ms=1e3 * fwd, backward_ms=1e3 * bwd, cores=cores,
                             kind="oracle", sample="100 y = A x and 20 backward passes "
                             "(explicit transpose each), Poisson 1000^2")
    if "eigsh" in nxt:
        rp, c, v = W.poisson_csr(N, np.int64)
        A = oracle.CSR(n, rp, c, v)
        m = 60
        t0 = time.perf_counter()
        oracle.lanczos(A, W.normal_rhs(n, 72), m)
        dt = time.perf_counter() - t0
        out["eigsh"] = dict(steps_per_s=m / dt, cores=cores, kind="oracle",
                            sample=f"{m} Lanczos steps (two Gram-Schmidt passes), Poisson "
                                   f"1000^2, {dt:.1f} s; the cost per step grows with the "
                                   "step index, so the 300-step rate is lower still")
    if "bicgstab" in nxt:
        rp, c, v = W.convection_diffusion_csr(N, rowptr_dtype=np.int64)
        A = oracle.CSR(n, rp, c, v)
        k = 500
        t0 = time.perf_counter()
        oracle.bicgstab(A, W.normal_rhs(n, 90), 0.0, k)
        dt = time.perf_counter() - t0
        out["bicgstab"] = dict(it_per_s=k / dt, cores=cores, kind="oracle",
                               sample=f"{k} BiCGStab iterations, convection-diffusion 1000^2, "
                                      f"{dt:.1f} s")
    if "list" in nxt:
        t0 = time.perf_counter()
        its = 0
        for i in range(8):
            Nl = 100 + 10 * i
            rp, c, v = W.poisson_csr(Nl, np.int64)
            _, info = oracle.cg(oracle.CSR(Nl * Nl, rp, c, v), W.uniform_rhs(Nl * Nl, i), 1e-8,
                                20000)
            its += info.iterations
        dt = time.perf_counter() - t0
        out["list"] = dict(systems_per_s=8 / dt, cores=cores, kind="oracle",
                           sample=f"the first 8 systems of the list (100^2 .. 170^2), "
                                  f"{its} CG iterations, {dt:.2f} s")
    return out


def cpu_baseline(seconds: float):
    """The oracle as it stands, on a bounded sample of the same workload:
    forward and adjoint CG on the 1000 x 1000 Poisson system, k fixed
    iterations each (k = 1000, the whole step, when one step fits in
    `seconds`), repeated whole steps until about `seconds` have passed."""
    import numpy as np
    import oracle
    import workloads as W
    _oracle_threads()
    N = 1000
    n = N * N
    rowptr, col, vals = W.poisson_csr(N, np.int64)
    A = oracle.CSR(n, rowptr, col, vals)
    _, b = W.manufactured(N)
    g = W.normal_rhs(n, 1)
    t0 = time.perf_counter()
    oracle.cg(A, b, 0.0, 5)
    per_it = (time.perf_counter() - t0) / 5
    k = int(max(5, min(1000, seconds / 2 / per_it)))
    steps = 0
    t0 = time.perf_counter()
    while True:
        x, fi = oracle.cg(A, b, 0.0, k)
        oracle.adjoint(A, x, g, 0.0, k)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or dt * (steps + 1) / steps > 2 * seconds:
            break
    return dict(value=2 * k * steps / dt, unit="CG iterations/s", cores=oracle.get_threads(),
                kind="oracle", cpu_model=oracle.cpu_model(), cpus_visible=os.cpu_count(),
                sample=f"Poisson 1000x1000 (n=1e6): {steps} x ({k} forward + {k} adjoint CG "
                       f"iterations with the pattern gradient), fp64, {dt:.1f} s")


def stream_ceiling(reps: int = 10) -> dict:
    """Bandwidth of plain stream kernels (torch's own element-wise and
    reduction kernels) on fp64 vectors of n = 16M and 169M elements: read
    (sum), R1W1 (copy), R2W1 (add), R3W1 (addcmul), each the median of
    `reps` event-timed launches after a warm-up.  At 16M the four vectors
    (512 MB) exceed the 256 MB Infinity Cache only twice over, at 169M
    (5.4 GB) every byte comes from HBM."""
    import numpy as np
    import torch
    out = {"peak_GBps": HBM_PEAK_GBPS}
    for n in (16_000_000, 169_000_000):
        a, b, c, d = (torch.rand(n, dtype=torch.float64, device="cuda") for _ in range(4))
        ops = {"read (sum)": (lambda: torch.sum(a), 1, 0),
               "R1W1 (copy)": (lambda: d.copy_(a), 1, 1),
               "R2W1 (add)": (lambda: torch.add(a, b, out=d), 2, 1),
               "R3W1 (addcmul)": (lambda: torch.addcmul(a, b, c, out=d), 3, 1)}
        res = {}
        for name, (fn, r, w) in ops.items():
            fn()
            torch.cuda.synchronize()
            ms = []
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            t = float(np.median(ms))
            res[name] = dict(ms=t, GBps=(r + w) * 8 * n / (t * 1e-3) / 1e9)
            log(f"[bench] stream n={n} {name}: {res[name]['GBps']:.0f} GB/s")
        out[f"n{n}"] = res
        del a, b, c, d
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--sizes", default="16m,169m,rgg4m,batch64,poisson32",
                    help="extra workloads: 16m / 169m (Poisson, 500 fixed iterations), rgg4m "
                         "(random geometric graph, tol 1e-8 forward + adjoint), batch64 (64 "
                         "Poisson 128^2 systems on one pattern), poisson32 (32^2, tol 1e-10, "
                         "and 256 such systems); '' for none; with "
                         "--skip-headline also matvec, eigsh, bicgstab, list and head (the "
                         "headline's forward solves alone)")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the .matvec and .eigsh measurements")
    ap.add_argument("--eig-steps", type=int, default=300,
                    help="Lanczos steps of the .eigsh measurement")
    ap.add_argument("--skip-headline", action="store_true",
                    help="only the --sizes runs (for profiler passes); prints no JSON line")
    ap.add_argument("--csr-only", action="store_true",
                    help="force the plain CSR kernels (no banded-pattern kernels)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only measure what plain element-wise stream kernels (torch's sum, "
                         "copy, add, addcmul) reach on fp64 vectors of the 16M and 169M "
                         "workloads' size: the practical bandwidth for each read/write mix; "
                         "prints one JSON line of its own and exits")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy a 1 GiB fp64 tensor 5 times (a plain copy kernel of known "
                         "size, to scale the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the solvers run "
              "on one GPU; sharding a system across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)
    global CSR_ONLY
    CSR_ONLY = args.csr_only
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import krylov_solvers_adjoint_amd  # noqa: F401  (fails loudly without the HIP library)

    if args.stream_ceiling:
        print(json.dumps(stream_ceiling()), flush=True)
        return
    if args.calibrate_copy:
        src = torch.ones(1 << 27, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        log(f"[bench] calibration copy: 1 GiB read + 1 GiB written per launch, "
            f"{2 * src.numel() * 8 / dt / 1e9:.0f} GB/s")
        del src, dst
    if args.skip_headline:
        for s in [s for s in args.sizes.split(",") if s]:
            import numpy as np
            if s.lower() == "rgg4m":
                out = bench_rgg(4_000_000, args.kernel_reps)
                log(f"[bench] rgg4m: {out}")
                continue
            if s.lower() == "matvec":
                log(f"[bench] matvec: {bench_matvec(args.kernel_reps)}")
                continue
            if s.lower() == "next16m":
                log(f"[bench] matvec 16M: {bench_matvec(args.kernel_reps, 4000)}")
                log(f"[bench] eigsh 16M: {bench_eigsh(60, 4, 4000)}")
                log(f"[bench] bicgstab 16M: {bench_bicgstab(4000, fixed=200)}")
                continue
            if s.lower() == "list":
                log(f"[bench] list: {bench_list()}")
                continue
            if s.lower() == "batch64":
                log(f"[bench] batch64: {bench_batch64(args.kernel_reps)}")
                continue
            if s.lower() == "poisson32":
                log(f"[bench] poisson32: {bench_poisson32()}")
                continue
            if s.lower() == "bicgstab":
                log(f"[bench] bicgstab: {bench_bicgstab()}")
                continue
            if s.lower() == "head":
                log(f"[bench] head: {bench_head_solves(5)}")
                continue
            if s.lower() == "eigsh":
                out = bench_eigsh(args.eig_steps, 4)
                log(f"[bench] eigsh: {out['ms']:.1f} ms, {out['eff_GBps']:.0f} GB/s")
                continue
            N, rp = {"1m": (1000, np.int32), "16m": (4000, np.int32),
                     "169m": (13000, np.int64)}[s.lower()]
            out = bench_size(N, rp, 500, args.kernel_reps, runs=1, warmups=1)[0]
            log(f"[bench] size {s}: {out['ms_per_iteration']:.3f} ms/it, "
                f"{out['canonical_GBps']:.0f} GB/s canonical, kernels {out['kernel_ms']}")
        return
    log(f"[bench] headline: Poisson 1000x1000, 1000 fwd + 1000 adj iterations, "
        f"{args.warmup} warm-up + {args.steps} timed steps")
    head = bench_headline(args)
    log(f"[bench] headline done: {head['ms_per_step']:.2f} ms/step, "
        f"{head['it_per_s']:.0f} it/s, kernels {head['kernel_ms']}")
    sizes = {}
    for s in [s for s in args.sizes.split(",") if s]:
        import numpy as np
        if s.lower() == "poisson32":
            log("[bench] size poisson32: 32x32 Poisson, tol 1e-10, forward + adjoint")
            sizes["poisson32"] = bench_poisson32()
            if not args.no_cpu:
                sizes["poisson32"]["cpu_1thread"] = oracle_poisson32()
            og, tk = sizes["poisson32"]["one_group"], sizes["poisson32"]["two_kernel"]
            log(f"[bench] size poisson32: {og['solve_adjoint_ms']:.3f} ms one workgroup, "
                f"{tk['solve_adjoint_ms']:.3f} ms two-kernel loop; 256 systems "
                f"{og['batch256_ms']:.3f} / {tk['batch256_ms']:.3f} ms")
            continue
        if s.lower() == "batch64":
            log("[bench] size batch64: 64 Poisson 128x128 systems, shared pattern, tol 1e-8")
            sizes["batch64"] = bench_batch64(args.kernel_reps)
            log(f"[bench] size batch64: {sizes['batch64']['us_per_step']:.1f} us per step")
            if not args.no_cpu:
                sizes["batch64"]["cpu_1thread"] = oracle_batch64()
            continue
        if s.lower() == "rgg4m":
            log("[bench] size rgg4m: random geometric graph, 4M nodes, tol 1e-8 fwd + adj")
            sizes["rgg4m"] = bench_rgg(4_000_000, args.kernel_reps)
            log(f"[bench] size rgg4m: {sizes['rgg4m']['iterations_fwd']}+"
                f"{sizes['rgg4m']['iterations_adj']} iterations, "
                f"{sizes['rgg4m']['it_per_s']:.0f} it/s, {sizes['rgg4m']['eff_GBps']:.0f} GB/s")
            ro = sizes["rgg4m"]["reordered"]
            log(f"[bench] size rgg4m reordered ({ro['order_ms']:.0f} ms to order): "
                f"{ro['iterations_fwd']}+{ro['iterations_adj']} iterations, "
                f"{ro['it_per_s']:.0f} it/s, {ro['eff_GBps']:.0f} GB/s")
            if not args.no_cpu:
                log("[bench] size rgg4m: the oracle's CSR build and a CG sample")
                sizes["rgg4m"]["cpu"] = oracle_rgg(4_000_000)
            continue
        N, rp = {"1m": (1000, np.int32), "16m": (4000, np.int32),
                 "169m": (13000, np.int64)}[s.lower()]
        log(f"[bench] size {s}: Poisson {N}x{N}, 500 fixed iterations, median of 5 after 2 warm-ups")
        out, b_np, x_np = bench_size(N, rp, 500, args.kernel_reps)
        sizes[s.lower()] = out
        ro = out["roofline"]
        log(f"[bench] size {s}: {out['ms_per_iteration']:.3f} ms/it, "
            f"{out['canonical_GBps']:.0f} GB/s canonical (frac {ro['frac_canonical']:.3f}), "
            f"iteration on moved bytes {ro.get('frac_iteration_moved')}")
        if not args.no_cpu:
            log(f"[bench] size {s}: the oracle's CG, 500 iterations on all host threads")
            out["cpu"] = oracle_fixed(N, rp, b_np, x_np)
            log(f"[bench] size {s}: oracle {out['cpu']['cpu_ms']:.0f} ms, x rel "
                f"{out['cpu']['oracle_rel_x']:.2e}")
            if s.lower() == "16m":
                out["cpu_1thread"] = oracle_one_thread_poisson(N, 10)
        del b_np, x_np

    nxt = {}
    if not args.no_next:
        log("[bench] .matvec on Poisson 1000x1000")
        nxt["matvec"] = bench_matvec(args.kernel_reps)
        log(f"[bench] .matvec: {nxt['matvec']}")
        log(f"[bench] .eigsh on Poisson 1000x1000: k=4 largest, {args.eig_steps} Lanczos steps")
        nxt["eigsh"] = bench_eigsh(args.eig_steps, 4)
        log(f"[bench] .eigsh: {nxt['eigsh']['ms']:.1f} ms, "
            f"{nxt['eigsh']['eff_GBps']:.0f} GB/s")
        log("[bench] BiCGStab on convection-diffusion 1000x1000, tol 1e-8, fwd + adj")
        nxt["bicgstab"] = bench_bicgstab()
        log(f"[bench] BiCGStab: {nxt['bicgstab']}")
        log("[bench] SparseTensorList: 32 Poisson grids 100^2 .. 410^2, CG tol 1e-8")
        nxt["list"] = bench_list()
        log(f"[bench] list: {nxt['list']}")
        # the same operations at 4000^2 (16M unknowns), where every byte comes
        # from HBM
        log("[bench] .matvec, .eigsh (60 steps) and BiCGStab (200 + 200 fixed iterations) "
            "at 4000x4000")
        nxt["matvec_16m"] = bench_matvec(args.kernel_reps, 4000)
        nxt["eigsh_16m"] = bench_eigsh(60, 4, 4000)
        nxt["bicgstab_16m"] = bench_bicgstab(4000, fixed=200)
        log(f"[bench] 16M: matvec {nxt['matvec_16m']['spmv_GBps']:.0f} / "
            f"{nxt['matvec_16m']['transpose_GBps']:.0f} / {nxt['matvec_16m']['backward_GBps']:.0f} "
            f"GB/s, eigsh {nxt['eigsh_16m']['eff_GBps']:.0f} GB/s, BiCGStab "
            f"{nxt['bicgstab_16m']['eff_GBps']:.0f} GB/s")

    digest = source_digest()
    ms_it = head["ms_per_step"] / (head["iterations_fwd"] + head["iterations_adj"])
    b_it = canonical_bytes(head["n"], head["nnz"], 4)
    if head["loop"] == "resident":
        # one launch runs all 1000 iterations of a solve; its algorithmic
        # bytes are the canonical bytes of those iterations
        loop_ms = head["loop_ms"]
        alg = head["loop_iterations"] * b_it
        achieved = alg / (loop_ms * 1e-3) / 1e9
        roofline = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=achieved / HBM_PEAK_GBPS,
                        traffic=traffic_from_profile("k_cg_grid", "poisson1000", digest),
                        kernel="k_cg_grid (the resident CG loop: a whole 1000-iteration solve "
                               "in one cooperative launch, the system held in registers and LDS)",
                        kernel_ms=loop_ms, algorithmic_bytes=alg,
                        iterations_per_launch=head["loop_iterations"],
                        us_per_iteration=1e3 * loop_ms / head["loop_iterations"],
                        source_digest=digest,
                        note="the loop reads the matrix once per launch and per iteration moves "
                             "only halo rows and the partial sums between workgroups, so the "
                             "canonical bytes a streaming iteration moves (12 nnz + 4 (n+1) + "
                             "88 n) exceed what HBM could deliver in its time (frac > 1); "
                             "traffic is what the counters saw per launch.  It is bound by the "
                             "latency of its one grid-wide sum per iteration (single-reduction "
                             "CG) and the on-chip SpMV, not by HBM; sizes.16m / sizes.169m "
                             "carry the HBM-bound rooflines of the two-kernel loop")
        if roofline["traffic"]:
            roofline["frac_kernel_moved"] = roofline["traffic"] / (loop_ms * 1e-3) / 1e9 / \
                HBM_PEAK_GBPS
    else:
        spmv_ms = head["kernel_ms"]["spmv_step"]
        achieved = head["spmv_bytes"] / (spmv_ms * 1e-3) / 1e9
        kname = STEP_KERNEL[head["spmv"]]
        roofline = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=achieved / HBM_PEAK_GBPS,
                        traffic=traffic_from_profile(kname, "poisson1000", digest),
                        kernel=f"{kname} ({head['spmv']}: SpMV + direction update + deferred x "
                               "update + p.Ap partials)",
                        kernel_ms=spmv_ms, algorithmic_bytes=head["spmv_bytes"],
                        source_digest=digest,
                        note="1M working set (about 110 MB) fits the 256 MB Infinity Cache: the "
                             "counted traffic leaves the L2 and is mostly served there, not by "
                             "HBM; sizes.16m / sizes.169m carry the HBM-resident rooflines")
        if roofline["traffic"]:
            roofline["frac_kernel_moved"] = roofline["traffic"] / (spmv_ms * 1e-3) / 1e9 / \
                HBM_PEAK_GBPS
    # as in the size legs: the whole iteration on canonical bytes
    roofline["frac_canonical"] = b_it / (ms_it * 1e-3) / 1e9 / HBM_PEAK_GBPS
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(args.cpu_seconds)
        # the same system on one thread, a bounded sample
        cpu["one_thread"] = oracle_one_thread_poisson(1000, 100)
        if nxt:
            log("[bench] CPU oracle beside the NEXT legs")
            for key, val in oracle_next(nxt).items():
                nxt[key]["cpu_oracle"] = val
    line = {
        "metric": METRIC,
        "value": head["it_per_s"],
        "unit": "CG iterations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "poisson1000_fixed1000_fwd_adj", "grid": "1000x1000",
                   "n": head["n"], "nnz": head["nnz"], "index": "i32/i32",
                   "loop": head["loop"], "spmv": head["spmv"],
                   "iterations_fwd": head["iterations_fwd"],
                   "iterations_adj": head["iterations_adj"], "parallelism": "none (1 GPU)"},
        "eff_GBps": head["eff_GBps"],
        "pct_peak_effective": head["pct_peak_effective"],
        "bandwidth_note": "eff_GBps: canonical bytes (12 nnz + 4 (n+1) + 88 n per iteration, "
                          "plus the pattern gradient) over the step's wall time; the resident "
                          "loop holds the 1M system on chip (the two-kernel loop's working set "
                          "is Infinity-Cache resident), so this is an effective rate, not HBM "
                          "bandwidth",
        "solution_rel_error": head["solution_rel_error"],
        "free_delta_MB": head["free_delta_MB"],
        "library_MB": head["library_MB"],
        "library_peak_MB": head["library_peak_MB"],
        "caller_MB": head["caller_MB"],
        "kernel_ms_two_kernel_loop": head["kernel_ms"],
        "forward_ms": head["forward_ms"],
        "adjoint_ms": head["adjoint_ms"],
        "pattern_grad": head["pattern_grad"],
        "roofline": roofline,
        "sizes": sizes,
        "next": nxt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
