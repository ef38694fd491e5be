"""Benchmark: PageRank power iteration on one MI355X.

One step = the whole path on one synthetic graph already resident in device
memory: pr_plan_create (vertices renumbered by degree bucket and out-degree,
inverse out-degrees, the in-edges sorted into tiles by the device
counting-sort machinery, the work units) and pr_run with 50 fixed iterations
(tol = 0, the timed mode of the Day 40 page).  The stand-alone pr_transpose of
the caller's graph is timed on its own.  The default workload is R-MAT scale
23, edge factor 32, (a, b, c, d) = (.57, .19, .19, .05), seed 23, self-loops
and duplicates removed.

Printed (one JSON line): whole-step throughput in GTEPS (edges x iterations /
step time); the per-iteration time and GTEPS; the gather-and-accumulate
kernel (k_tile, timed launch by launch with events on the run's stream)
against the HBM roofline, counting the bytes any pull iteration must move,
beside the counter-measured traffic and Day 40's own byte model; the
L1 < 1e-6 run; the other workloads (citation-like, 27-point stencil, R-MAT
18 and 21, and R-MAT 23 with shuffled ids); the rerun after an edge batch;
and the CPU oracle's rate on a bounded sample of the same graph, on one
pinned core, with the host's CPU model and core count.

    python bench.py [--steps K] [--warmup W] [--workload rmat23] [--iters 50]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
MAIN_KERNEL = "k_tile"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "k_tile_rmat23_counters.json")
# the kernel and the plan code that lays out its tiles and units
KERNEL_SOURCES = ["pagerank_power_iteration_amd/csrc/run.hip",
                  "pagerank_power_iteration_amd/csrc/plan.hip",
                  "pagerank_power_iteration_amd/csrc/plan.hpp",
                  "pagerank_power_iteration_amd/csrc/radix.hpp",
                  "pagerank_power_iteration_amd/csrc/common.hpp"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def min_bytes_per_iteration(n: int, m: int) -> int:
    """Bytes any pull iteration must move: per edge a 4-byte column index and a
    4-byte gathered contribution; per vertex row_ptr, x read, x' write,
    inverse out-degree and contrib' write (4 bytes each); plus row_ptr[n]."""
    return 8 * m + 20 * n + 4


def day40_hand_bytes(n: int, m: int) -> int:
    """Day 40's own byte count of one iteration of its hand-written kernels
    ("Results"): scale 12n, SpMV 8m + 8n + 4, dangling 5n, residual 8n,
    combine 8n, i.e. 33n + 8m + 4 (3,437,470 bytes on its citation graph)."""
    return 33 * n + 8 * m + 4


def traffic_from_counters(n_launch_bytes: int):
    """HBM bytes per k_tile launch from the committed rocprofv3 counter
    summary, when it was taken on the current kernel and plan source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None, c.get("kernel_source_hash")
    return c.get("hbm_bytes_per_launch"), c.get("kernel_source_hash")


def copy_row(torch, gib: float = 2.0, reps: int = 5) -> float:
    """Device-to-device copy bandwidth (read + write bytes) of a buffer larger
    than the 256 MB Infinity Cache."""
    nbytes = int(gib * (1 << 30))
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_traversal_baseline(g) -> dict:
    """The oracle's breadth-first search from vertex 0 and weak components on
    the same graph, single-threaded, search loops only."""
    import oracle
    with pinned_to_one_core():
        ref = oracle.bfs(g.row_ptr, g.col_idx, 0)
        _, _, wcc_secs = oracle.wcc(g.row_ptr, g.col_idx, timed=True)
    return {"bfs_ms": round(ref.loop_seconds * 1e3, 2),
            "bfs_gteps": round(ref.edges_scanned / ref.loop_seconds / 1e9, 4),
            "wcc_ms": round(wcc_secs * 1e3, 2), "wcc_gteps": round(g.m / wcc_secs / 1e9, 4),
            "cores": 1}


def cpu_spmv_baseline(graphgen, nx: int) -> dict:
    """The oracle's product loop on the same seeded stencil matrix as the
    GPU leg, single-threaded."""
    import oracle
    A = graphgen.stencil_matrix(nx, values="random", seed=5)
    x = graphgen.uniform(A.n_cols, 6)
    with pinned_to_one_core():
        _, secs = oracle.spmv(A.row_ptr, A.col_idx, A.vals, x, A.n_cols, timed=True)
    return {"ms": round(secs * 1e3, 2), "gflops": round(2 * A.nnz / secs / 1e9, 3), "cores": 1}


def host_info() -> dict:
    """The host the CPU baseline runs on: CPU model, logical CPUs, and the
    CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = sorted(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = []
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": _ranges(allowed)}


def _ranges(cpus) -> str:
    out, i = [], 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(f"{cpus[i]}" if i == j else f"{cpus[i]}-{cpus[j]}")
        i = j + 1
    return ",".join(out)


class pinned_to_one_core:
    """Run the calling thread on one CPU (the last one it may use), then
    restore its affinity.  The oracle runs in this thread through ctypes, so
    it is pinned too."""

    def __enter__(self):
        self.before = None
        self.core = None
        try:
            self.before = os.sched_getaffinity(0)
            self.core = max(self.before)
            os.sched_setaffinity(0, {self.core})
        except (AttributeError, OSError):
            pass
        return self

    def __exit__(self, *exc):
        if self.before is not None:
            os.sched_setaffinity(0, self.before)
        return False


def cpu_baseline(g, iters: int) -> dict:
    import oracle
    with pinned_to_one_core() as pin:
        r = oracle.pagerank(g.row_ptr, g.col_idx, d=0.85, tol=0.0, max_iter=iters)
    secs = r.loop_seconds
    return {"value": round(g.m * iters / secs / 1e9, 4), "unit": "GTEPS", "cores": 1,
            "kind": "oracle",
            "sample": f"{iters} of the 50 iterations on the same {g.name} graph "
                      f"(fp64, single thread pinned to CPU {pin.core}, iteration loop only: "
                      f"{secs:.2f} s)",
            "ms_per_iteration": round(secs * 1e3 / iters, 2), "pinned_cpu": pin.core,
            "host": host_info()}


def spmv_min_bytes(n_rows: int, n_cols: int, nnz: int) -> int:
    """Bytes any CSR product y = A x in double must move: per stored entry a
    4-byte column index and an 8-byte value; per row a row pointer and the
    8-byte y; each x entry once; plus row_ptr[n_rows]."""
    return 12 * nnz + 12 * n_rows + 8 * n_cols + 4


def spmv_rate(torch, prx, graphgen, nx: int, reps: int) -> dict:
    """The valued fp64 product of the 27-point stencil operator (diagonal
    stored) on an nx^3 grid with seeded uniform values: plan once, one
    warm-up product, then `reps` products timed together with events on the
    stream they are launched on."""
    A = graphgen.stencil_matrix(nx, values="random", seed=5)
    x = graphgen.uniform(A.n_cols, 6)
    plan = prx.SpmvPlan.from_csr(A.row_ptr, A.col_idx, A.n_cols)
    vals = torch.as_tensor(A.vals, dtype=torch.float64).cuda()
    xd = torch.as_tensor(x, dtype=torch.float64).cuda()
    y = torch.empty(A.n_rows, dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()
    plan.run(vals, xd, y, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(3):
        e0.record(stream)
        for _ in range(reps):
            plan.run(vals, xd, y, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    ms = statistics.median(times)
    b = spmv_min_bytes(A.n_rows, A.n_cols, A.nnz)
    items = plan.items()
    plan.close()
    return {"workload": A.name, "n_rows": A.n_rows, "nnz": A.nnz, "dtype": "f64",
            "launch_ms": round(ms, 5), "gflops": round(2 * A.nnz / (ms * 1e-3) / 1e9, 1),
            "algorithmic_bytes": b, "gbps": round(b / (ms * 1e-3) / 1e9, 1),
            "frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "items": items}


def bfs_min_bytes(n: int, scanned: int, reached: int) -> int:
    """Bytes a top-down breadth-first search must move: per scanned edge a
    4-byte column and a 4-byte level read; per reached vertex its two row
    pointers, its frontier-queue write and read and its level write; the level
    array initialised once."""
    return 8 * scanned + 20 * reached + 4 * n


def wcc_min_bytes(n: int, m: int) -> int:
    """Bytes a one-pass linking of weak components must move: per edge a
    4-byte column and a 4-byte label read; per vertex the label initialised,
    its row pointer, its own label read, and the final pass's read and write."""
    return 8 * m + 20 * n


def traversal_rates(torch, prx, g, dg, reps: int = 5) -> dict:
    """BFS from vertex 0 and weak components on one resident graph, given
    its in-edge CSR from pr_transpose (bottom-up levels, giant-tree skip) and
    without it: median of `reps` timed calls after one warm-up, each call
    bracketed by device synchronizations (pr_bfs synchronizes its stream
    itself).  The transpose is built once, outside the timed calls."""
    stream = torch.cuda.current_stream()
    in_rp, in_ci = prx.transpose(dg)
    level = torch.empty(g.n, dtype=torch.int32, device="cuda")
    label = torch.empty(g.n, dtype=torch.int32, device="cuda")
    ws_b = torch.empty(prx.pr_bfs_workspace_bytes(g.n, g.m), dtype=torch.uint8, device="cuda")
    ws_w = torch.empty(prx.pr_wcc_workspace_bytes(g.n, g.m), dtype=torch.uint8, device="cuda")

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            out = fn()
            torch.cuda.synchronize()
            ts.append((time.perf_counter() - t0) * 1e3)
        return statistics.median(ts), out

    def bfs(irp, ici):
        return prx.pr_bfs(g.n, g.m, dg.row_ptr, dg.col_idx, 0, level, ws_b, irp, ici, 0, stream)

    def wcc(irp, ici):
        return prx.pr_wcc(g.n, g.m, dg.row_ptr, dg.col_idx, label, ws_w, irp, ici, 0, stream,
                          count_components=True)

    bfs_out_ms, _ = timed(lambda: bfs(None, None))
    wcc_out_ms, _ = timed(lambda: wcc(None, None))
    bfs_ms, (depth, scanned) = timed(lambda: bfs(in_rp, in_ci))
    reached = int((level >= 0).sum().item())
    wcc_ms, comps = timed(lambda: wcc(in_rp, in_ci))
    bb = bfs_min_bytes(g.n, scanned, reached)
    wb = wcc_min_bytes(g.n, g.m)
    return {
        "bfs": {"source": 0, "ms": round(bfs_ms, 4), "depth": depth, "reached": reached,
                "edges_scanned": scanned, "gteps": round(scanned / (bfs_ms * 1e-3) / 1e9, 2),
                "algorithmic_bytes": bb, "gbps": round(bb / (bfs_ms * 1e-3) / 1e9, 1),
                "frac": round(bb / (bfs_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "out_edges_only_ms": round(bfs_out_ms, 4)},
        "wcc": {"ms": round(wcc_ms, 4), "components": comps,
                "gteps": round(g.m / (wcc_ms * 1e-3) / 1e9, 2), "algorithmic_bytes": wb,
                "gbps": round(wb / (wcc_ms * 1e-3) / 1e9, 1),
                "frac": round(wb / (wcc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "out_edges_only_ms": round(wcc_out_ms, 4)},
    }


def iteration_ms(torch, prx, plan, n: int, iters: int, reps: int = 5) -> float:
    """Milliseconds per iteration of a fixed-iteration pr_run, with no timing
    events between its launches (on small graphs an event pair around each
    launch costs as much as the launch): the median over `reps` of the time of
    a 2*iters run minus that of an iters run, over iters, so the run's
    one-time kernels (start vector in, ranks out, last reduction) cancel."""
    stream = torch.cuda.current_stream()
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    l1 = torch.empty(2 * iters, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(k):
        e0.record(stream)
        prx.pr_run(plan, 0.85, 0.0, k, x, l1, None, 0, stream)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1)

    run(iters)
    diffs = []
    for _ in range(reps):
        short = run(iters)
        diffs.append((run(2 * iters) - short) / iters)
    return statistics.median(diffs)


def workload_rate(torch, prx, graphgen, name: str, iters: int) -> dict:
    """Per-iteration rate of one more workload: a plan (timed), one warm-up
    run, the time per iteration (iteration_ms) and the gather kernel's mean
    launch time (event pairs around each launch, a separate run) against the
    same roofline."""
    t0 = time.time()
    g = graphgen.workload(name)
    log(f"{name}: n={g.n} m={g.m} generated in {time.time() - t0:.1f}s")
    dg = prx.DeviceGraph.from_csr(g.row_ptr, g.col_idx)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prx.Plan(dg).close()  # warm-up plan
    torch.cuda.synchronize()
    e0.record(stream)
    plan = prx.Plan(dg)
    e1.record(stream)
    torch.cuda.synchronize()
    plan_ms = e0.elapsed_time(e1)
    plan.run(max_iter=3)
    it = iteration_ms(torch, prx, plan.handle, g.n, iters)
    kms = []
    for _ in range(3):
        plan.run(max_iter=iters, record_events=True)
        kms.append(plan.kernel_ms()[0])
    plan.close()
    km = statistics.median(kms)
    b = min_bytes_per_iteration(g.n, g.m)
    hb = day40_hand_bytes(g.n, g.m)
    cached = b < 256e6
    return {"n": g.n, "m": g.m, "plan_ms": round(plan_ms, 4), "iteration_ms": round(it, 5),
            "gteps": round(g.m / (it * 1e-3) / 1e9, 2), "kernel_ms": round(km, 5),
            "roofline_frac": round(b / (km * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "iteration_frac": round(b / (it * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "day40_model_frac": round(hb / (it * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": ("working set fits the 256 MB Infinity Cache: not an HBM point" if cached
                     else "working set exceeds the Infinity Cache")}


def incremental_rate(torch, prx, graphgen, g, dg, iters_cap: int = 200, tol: float = 1e-6) -> dict:
    """The rerun after an edge batch (Meerkat's incremental/decremental
    PageRank): ranks of G to tol, then a seeded batch (m/256 deletions of
    existing edges and m/256 R-MAT insertion draws) gives G', which is
    re-planned and iterated to tol twice: from G's ranks (warm) and from 1/n
    (cold).  The batch is applied on the host and G' uploaded before anything
    is timed."""
    stream = torch.cuda.current_stream()
    plan = prx.Plan(dg)
    before = plan.run(tol=tol, max_iter=iters_cap)
    x_g = before.x.clone()
    plan.close()
    del plan
    t0 = time.time()
    dele, u, v = graphgen.edge_batch(g, g.m // 256, g.m // 256, seed=256)
    g2 = graphgen.apply_batch(g, dele, u, v)
    log(f"edge batch: -{dele.size} / +{u.size} draws, m {g.m} -> {g2.m} ({time.time() - t0:.1f}s)")
    dg2 = prx.DeviceGraph.from_csr(g2.row_ptr, g2.col_idx)
    ws = torch.empty(prx.pr_plan_workspace_bytes(g2.n, g2.m), dtype=torch.uint8, device="cuda")
    scratch = torch.empty(prx.pr_plan_scratch_bytes(g2.n, g2.m), dtype=torch.uint8, device="cuda")
    x = torch.empty(g2.n, dtype=torch.float32, device="cuda")
    l1 = torch.empty(iters_cap, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    replans = []
    for _ in range(3):
        torch.cuda.synchronize()
        e0.record(stream)
        h = prx.pr_plan_create(g2.n, g2.m, dg2.row_ptr, dg2.col_idx, ws, scratch, 0, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        replans.append(e0.elapsed_time(e1))
        prx.pr_plan_destroy(h)
    h = prx.pr_plan_create(g2.n, g2.m, dg2.row_ptr, dg2.col_idx, ws, scratch, 0, stream)

    def run(warm: bool):
        if warm:
            x.copy_(x_g)
        torch.cuda.synchronize()
        t = time.perf_counter()
        it = prx.pr_run(h, 0.85, tol, iters_cap, x, l1, None,
                        prx.PR_X0_GIVEN if warm else 0, stream)
        torch.cuda.synchronize()
        return it, (time.perf_counter() - t) * 1e3

    run(True)
    it_warm, ms_warm = run(True)
    it_cold, ms_cold = run(False)
    prx.pr_plan_destroy(h)
    return {"graph": g.name, "batch_delete": int(dele.size), "batch_insert_draws": int(u.size),
            "m_before": g.m, "m_after": g2.m, "tol": tol, "iters_before": before.iterations,
            "replan_ms": round(statistics.median(replans), 4), "iters_warm": it_warm,
            "warm_ms": round(ms_warm, 3), "iters_cold": it_cold, "cold_ms": round(ms_cold, 3)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="rmat23")
    ap.add_argument("--iters", type=int, default=50)
    ap.add_argument("--cpu-iters", type=int, default=12,
                    help="iterations of the CPU oracle sample (0 skips it)")
    ap.add_argument("--no-copy-row", action="store_true")
    ap.add_argument("--spmv-grid", type=int, default=100,
                    help="edge of the 27-point stencil grid of the valued fp64 product "
                         "(0 skips it)")
    ap.add_argument("--traversal", default="rmat23,grid1024",
                    help="graphs on which BFS from vertex 0 and weak components are timed "
                         "(the main workload's graph is reused when named; empty skips)")
    ap.add_argument("--workloads", default="citation,stencil100,rmat18,rmat21,rmat23r",
                    help="comma-separated extra workloads whose plan time and per-iteration "
                         "rate are added under 'workloads' (rmat23r: R-MAT 23 with seeded "
                         "shuffled ids; empty skips)")
    ap.add_argument("--no-incremental", action="store_true",
                    help="skip the rerun after an edge batch")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import graphgen
    import pagerank_power_iteration_amd as prx

    prx.lib()
    torch.cuda.set_device(0)
    t0 = time.time()
    g = graphgen.workload(args.workload)
    n, m = g.n, g.m
    log(f"{g.name}: n={n} m={m} generated in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    dg = prx.DeviceGraph.from_csr(g.row_ptr, g.col_idx)
    ws_p = torch.empty(prx.pr_plan_workspace_bytes(n, m), dtype=torch.uint8, device="cuda")
    scratch = torch.empty(prx.pr_plan_scratch_bytes(n, m), dtype=torch.uint8, device="cuda")
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    l1 = torch.empty(args.iters, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def step():
        ev[0].record(stream)
        plan = prx.pr_plan_create(n, m, dg.row_ptr, dg.col_idx, ws_p, scratch, 0, stream)
        ev[1].record(stream)
        prx.pr_run(plan, 0.85, 0.0, args.iters, x, l1, None, 0, stream)
        ev[2].record(stream)
        ev[2].synchronize()  # the step ends when its ranks are back in the caller's order
        prx.pr_plan_destroy(plan)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    parts = {"plan": [], "run": []}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
        parts["plan"].append(ev[0].elapsed_time(ev[1]))
        parts["run"].append(ev[1].elapsed_time(ev[2]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    med = {k: statistics.median(v) for k, v in parts.items()}

    # outside the timed steps: the time per iteration without timing events
    # between launches, and the gather kernel's launch time (an event pair on
    # the run's stream around each of its first 64 launches)
    plan = prx.pr_plan_create(n, m, dg.row_ptr, dg.col_idx, ws_p, scratch, 0, stream)
    med["iter"] = iteration_ms(torch, prx, plan, n, args.iters)
    kms = []
    for _ in range(3):
        prx.pr_run(plan, 0.85, 0.0, args.iters, x, l1, None, prx.PR_RECORD_EVENTS, stream)
        kms.append(prx.pr_plan_kernel_ms(plan)[0])
    med["kernel"] = statistics.median(kms)
    prx.pr_plan_destroy(plan)
    iter_runs = [r / args.iters for r in parts["run"]]

    # the caller-facing transpose, outside the step (its output is not used by the plan)
    del scratch
    in_rp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    in_ci = torch.empty(max(m, 1), dtype=torch.int32, device="cuda")[:m]
    ws_t = torch.empty(prx.pr_transpose_workspace_bytes(n, m), dtype=torch.uint8, device="cuda")
    tt = []
    for i in range(4):
        ev[0].record(stream)
        prx.pr_transpose(n, m, dg.row_ptr, dg.col_idx, in_rp, in_ci, ws_t, 0, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i:
            tt.append(ev[0].elapsed_time(ev[1]))
    med["transpose"] = statistics.median(tt)
    del ws_t, in_rp, in_ci
    iter_ms = med["iter"]
    kernel_ms = med["kernel"]
    bytes_iter = min_bytes_per_iteration(n, m)
    achieved = bytes_iter / (kernel_ms * 1e-3) / 1e9
    traffic, _ = traffic_from_counters(bytes_iter)
    log(f"step {ms_per_step:.3f} ms: plan {med['plan']:.3f} ms, run {med['run']:.3f} ms "
        f"({iter_ms * 1e3:.1f} us/iteration, {MAIN_KERNEL} {kernel_ms * 1e3:.1f} us/launch); "
        f"pr_transpose alone {med['transpose']:.3f} ms")

    scratch = torch.empty(prx.pr_plan_scratch_bytes(n, m), dtype=torch.uint8, device="cuda")
    plan = prx.pr_plan_create(n, m, dg.row_ptr, dg.col_idx, ws_p, scratch, 0, stream)
    buckets = prx.pr_plan_buckets(plan)
    # the convergence run of the same configuration: stop at the first
    # iteration whose L1 distance is below 1e-6 (at most 200 iterations)
    tol_l1 = torch.empty(200, dtype=torch.float32, device="cuda")
    prx.pr_run(plan, 0.85, 1e-6, 200, x, tol_l1, None, 0, stream)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tol_it = prx.pr_run(plan, 0.85, 1e-6, 200, x, tol_l1, None, 0, stream)
    torch.cuda.synchronize()
    tol_ms = (time.perf_counter() - t0) * 1e3
    tol_run = {"tol": 1e-6, "iterations": tol_it, "ms": round(tol_ms, 3),
               "final_l1": float(tol_l1[tol_it - 1].item()),
               "gteps": round(m * tol_it / (tol_ms * 1e-3) / 1e9, 2)}
    log(f"tolerance run: {tol_run}")
    prx.pr_plan_destroy(plan)
    del scratch, ws_p
    torch.cuda.empty_cache()
    copy_gbps = None if args.no_copy_row else round(copy_row(torch), 1)

    incremental = None
    if not args.no_incremental:
        incremental = incremental_rate(torch, prx, graphgen, g, dg)
        log(f"incremental: {incremental}")
        torch.cuda.empty_cache()

    extra = {}
    for name in [w for w in args.workloads.split(",") if w]:
        extra[name] = workload_rate(torch, prx, graphgen, name, args.iters)
        log(f"{name}: {extra[name]}")

    trav, trav_graphs = {}, {}
    for name in [w for w in args.traversal.split(",") if w]:
        if name == g.name:
            tg, tdg = g, dg
        else:
            tg = graphgen.workload(name)
            tdg = prx.DeviceGraph.from_csr(tg.row_ptr, tg.col_idx)
        trav[name] = traversal_rates(torch, prx, tg, tdg)
        trav_graphs[name] = tg
        log(f"traversal {name}: {trav[name]}")
        del tdg
    torch.cuda.empty_cache()

    spmv = None
    if args.spmv_grid > 0:
        spmv = spmv_rate(torch, prx, graphgen, args.spmv_grid, 50)
        log(f"spmv: {spmv}")

    cpu = None
    if args.cpu_iters > 0:
        log(f"timing the CPU oracle on {args.cpu_iters} iterations ...")
        cpu = cpu_baseline(g, args.cpu_iters)
        if trav_graphs:
            cpu["traversal"] = {k: cpu_traversal_baseline(v) for k, v in trav_graphs.items()}
        if args.spmv_grid > 0:
            cpu["spmv"] = cpu_spmv_baseline(graphgen, args.spmv_grid)

    iter_cv = (statistics.pstdev(iter_runs) / statistics.mean(iter_runs)
               if len(iter_runs) > 1 else 0.0)
    out = {
        "metric": "GTEPS per PageRank iteration + achieved HBM GB/s (% peak), RMAT scale 23",
        "value": round(m * args.iters / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "GTEPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": g.name, "n": n, "m": m, "iterations": args.iters, "d": 0.85,
                   "tol": 0.0, "index": "int32", "step": "pr_plan_create + pr_run"},
        "iteration": {"ms": round(iter_ms, 5), "gteps": round(m / (iter_ms * 1e-3) / 1e9, 2),
                      "gbps": round(bytes_iter / (iter_ms * 1e-3) / 1e9, 1),
                      "cv": round(iter_cv, 4), "algorithmic_bytes": bytes_iter,
                      "kernel_ms": round(kernel_ms, 5),
                      "basis": "(time of a 100-iteration run - time of a 50-iteration run) / 50, "
                               "no timing events between launches; cv over the timed steps' runs"},
        "transpose_ms": round(med["transpose"], 4),
        "transpose": {"ms": round(med["transpose"], 4),
                      "algorithmic_bytes": 8 * m + 8 * (n + 1),
                      "frac": round((8 * m + 8 * (n + 1)) / (med["transpose"] * 1e-3) / 1e9
                                    / HBM_PEAK_GBPS, 4),
                      "note": "bytes any transpose must move: read the out-edge CSR, write the "
                              "in-edge CSR"},
        "tol_run": tol_run,
        "plan_ms": round(med["plan"], 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": MAIN_KERNEL,
                     "launch_ms": round(kernel_ms, 5),
                     "achieved_basis": "algorithmic: B_min = 8m + 20n + 4 bytes (what any pull "
                                       "iteration must move) per launch / launch time",
                     "counter_gbps": (round(traffic / (kernel_ms * 1e-3) / 1e9, 1)
                                      if traffic else None),
                     "counter_frac": (round(traffic / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                                      if traffic else None),
                     "iteration_frac": round(bytes_iter / (iter_ms * 1e-3) / 1e9
                                             / HBM_PEAK_GBPS, 4)},
        "byte_models": {"b_min": bytes_iter, "b_min_frac_iteration":
                        round(bytes_iter / (iter_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "day40_hand_model": day40_hand_bytes(n, m),
                        "day40_hand_model_frac_iteration":
                        round(day40_hand_bytes(n, m) / (iter_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "note": "Day 40 counts 33n + 8m + 4 bytes per iteration of its "
                                "five-kernel design; B_min = 8m + 20n + 4 is the pull "
                                "minimum; counter traffic is what the L2s exchanged with "
                                "the fabric per gather launch"},
        "copy_row_gbps": copy_gbps,
        "buckets": buckets,
        "cpu_baseline": cpu,
    }
    if spmv:
        out["spmv"] = spmv
    if trav:
        out["traversal"] = trav
    if extra:
        out["workloads"] = extra
    if incremental:
        out["incremental"] = incremental
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
