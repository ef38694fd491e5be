"""PageRank power iteration with dangling-node redistribution on one AMD
Instinct MI355X (gfx950).

Every step runs in the HIP library ``libpr.so`` behind the C ABI in
``include/pr.h``; ``_lib`` binds it with ctypes under the same names.  The
helpers below only allocate device memory with torch and pass pointers:

    >>> import pagerank_power_iteration_amd as prx
    >>> g = prx.DeviceGraph.from_csr(row_ptr, col_idx)     # numpy int32 CSR
    >>> plan = prx.Plan(g)                                 # pr_plan_create
    >>> res = plan.run(d=0.85, tol=1e-6, max_iter=100)     # pr_run
    >>> res.x, res.iterations, res.l1_trace

The valued sparse product y = A x (fp64 CSR, pr_spmv):

    >>> A = prx.SpmvPlan.from_csr(row_ptr, col_idx, n_cols)  # pr_spmv_plan_create
    >>> y = A.run(vals, x)                                   # pr_spmv
"""
from __future__ import annotations

from ._lib import (PR_ERR_ARG, PR_ERR_GRAPH, PR_ERR_HIP, PR_ERR_WORKSPACE, PR_OK,
                   PR_PLAN_BUCKETED, PR_RECORD_EVENTS, PR_VALIDATE, PR_X0_GIVEN, PrError,
                   lib, pr_bfs, pr_bfs_workspace_bytes, pr_last_error, pr_wcc,
                   pr_wcc_workspace_bytes, pr_plan_buckets, pr_plan_create, pr_plan_destroy,
                   pr_plan_iteration_ms, pr_plan_kernel_ms, pr_plan_layout, pr_plan_tiles, pr_plan_num_buckets,
                   pr_plan_scratch_bytes, pr_plan_workspace_bytes, pr_run, pr_status_string,
                   pr_spmv, pr_spmv_plan_create, pr_spmv_plan_destroy, pr_spmv_plan_items,
                   pr_spmv_scratch_bytes, pr_spmv_workspace_bytes, pr_transpose,
                   pr_transpose_noalloc, pr_transpose_workspace_bytes,
                   PR_NOALLOC_SCRATCH_BYTES)

__all__ = [
    "DeviceGraph", "Plan", "RunResult", "transpose", "PrError", "lib",
    "pr_transpose", "pr_transpose_workspace_bytes", "pr_transpose_noalloc",
    "PR_NOALLOC_SCRATCH_BYTES", "pr_plan_create", "pr_plan_destroy",
    "pr_plan_workspace_bytes", "pr_plan_scratch_bytes", "pr_run", "pr_plan_iteration_ms",
    "pr_plan_kernel_ms", "pr_plan_tiles",
    "pr_plan_buckets", "pr_plan_num_buckets", "pr_plan_layout", "pr_status_string",
    "pr_last_error", "SpmvPlan", "pr_spmv", "pr_spmv_plan_create", "pr_spmv_plan_destroy",
    "pr_spmv_plan_items", "pr_spmv_scratch_bytes", "pr_spmv_workspace_bytes",
    "bfs", "wcc", "pr_bfs", "pr_bfs_workspace_bytes", "pr_wcc", "pr_wcc_workspace_bytes",
    "PR_OK", "PR_ERR_ARG", "PR_ERR_WORKSPACE", "PR_ERR_GRAPH", "PR_ERR_HIP",
    "PR_VALIDATE", "PR_PLAN_BUCKETED", "PR_X0_GIVEN", "PR_RECORD_EVENTS",
]


def _torch():
    import torch
    return torch


def _device_buffer(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class DeviceGraph:
    """Out-edge CSR resident in device memory (int32)."""

    def __init__(self, row_ptr, col_idx):
        self.row_ptr = row_ptr
        self.col_idx = col_idx
        self.n = int(row_ptr.numel() - 1)
        self.nnz = int(col_idx.numel())

    @classmethod
    def from_csr(cls, row_ptr, col_idx, device="cuda"):
        torch = _torch()
        rp = torch.as_tensor(row_ptr, dtype=torch.int32).to(device)
        ci = torch.as_tensor(col_idx, dtype=torch.int32).to(device)
        if ci.numel() == 0:
            ci = torch.zeros(1, dtype=torch.int32, device=device)[:0]
        return cls(rp, ci)


def transpose(graph: DeviceGraph, flags: int = 0, stream=None, ws=None):
    """In-edge CSR (in_row_ptr, in_col_idx) of `graph` via pr_transpose."""
    torch = _torch()
    dev = graph.row_ptr.device
    in_rp = torch.empty(graph.n + 1, dtype=torch.int32, device=dev)
    in_ci = torch.empty(max(graph.nnz, 1), dtype=torch.int32, device=dev)[: graph.nnz]
    if ws is None:
        ws = _device_buffer(pr_transpose_workspace_bytes(graph.n, graph.nnz), dev)
    pr_transpose(graph.n, graph.nnz, graph.row_ptr, graph.col_idx, in_rp, in_ci, ws, flags, stream)
    return in_rp, in_ci


def bfs(graph: DeviceGraph, source: int, in_csr=None, flags: int = 0, stream=None, ws=None,
        out=None):
    """Breadth-first levels from `source` via pr_bfs: (level int32[n] on the
    device, depth, out-edges scanned).  `in_csr` = (in_row_ptr, in_col_idx),
    e.g. transpose(graph), enables bottom-up levels."""
    torch = _torch()
    dev = graph.row_ptr.device
    level = out if out is not None else torch.empty(graph.n, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _device_buffer(pr_bfs_workspace_bytes(graph.n, graph.nnz), dev)
    irp, ici = in_csr if in_csr is not None else (None, None)
    depth, scanned = pr_bfs(graph.n, graph.nnz, graph.row_ptr, graph.col_idx, source, level, ws,
                            irp, ici, flags, stream)
    return level, depth, scanned


def wcc(graph: DeviceGraph, in_csr=None, flags: int = 0, stream=None, ws=None, out=None):
    """Weakly connected components via pr_wcc: (label int32[n] on the device,
    number of components).  `in_csr` lets the full pass skip the giant
    component."""
    torch = _torch()
    dev = graph.row_ptr.device
    label = out if out is not None else torch.empty(graph.n, dtype=torch.int32, device=dev)
    if ws is None:
        ws = _device_buffer(pr_wcc_workspace_bytes(graph.n, graph.nnz), dev)
    irp, ici = in_csr if in_csr is not None else (None, None)
    comps = pr_wcc(graph.n, graph.nnz, graph.row_ptr, graph.col_idx, label, ws, irp, ici, flags,
                   stream)
    return label, comps


class RunResult:
    __slots__ = ("x", "iterations", "l1_trace", "sum_trace")

    def __init__(self, x, iterations, l1_trace, sum_trace):
        self.x, self.iterations, self.l1_trace, self.sum_trace = x, iterations, l1_trace, sum_trace


class Plan:
    """A graph planned on the device (pr_plan_create), ready for pr_run.

    Keeps the plan's workspace alive for its lifetime; the out-edge CSR and
    the scratch buffer are only needed while it is built.
    """

    def __init__(self, graph: DeviceGraph, flags: int = 0, stream=None):
        self.graph = graph
        dev = graph.row_ptr.device
        self.ws = _device_buffer(pr_plan_workspace_bytes(graph.n, graph.nnz), dev)
        scratch = _device_buffer(pr_plan_scratch_bytes(graph.n, graph.nnz), dev)
        self.handle = pr_plan_create(graph.n, graph.nnz, graph.row_ptr, graph.col_idx, self.ws,
                                     scratch, flags, stream)
        del scratch

    def layout(self):
        """(in_row_ptr, in_col_idx, new_id) of the plan as torch tensors (views
        of the plan's workspace): the in-edge CSR in plan ids and the plan id
        of each of the caller's vertices."""
        torch = _torch()
        rp, ci, nid = pr_plan_layout(self.handle)
        base = self.ws.data_ptr()
        n, m = self.graph.n, self.graph.nnz

        def view(addr, count):
            off = addr - base
            return self.ws[off:off + 4 * count].view(torch.int32)
        return (None if rp is None else view(rp, n + 1)), (None if ci is None else view(ci, m)), \
            view(nid, n)

    def tiles(self):
        """Tiled plans: (tile_src int32[slots], tile_row int16[slots] (the row
        offset in its tile, as unsigned 16-bit; wide blocks only),
        tile_block int32[slots/256], tile_ptr int32[n_tiles+1], row0, rows)
        -- device views and numpy arrays.  Tile t owns slots
        [tile_ptr[t], tile_ptr[t+1]), its edges padded to whole blocks of
        256, each block stored transposed and narrow blocks packed (see
        pr_plan_tiles)."""
        torch = _torch()
        src, row, blk, ptr, nt, row0, rows = pr_plan_tiles(self.handle)
        base = self.ws.data_ptr()

        def view(addr, nbytes, dtype):
            off = addr - base
            return self.ws[off:off + nbytes].view(dtype)
        tile_ptr = view(ptr, 4 * (nt + 1), torch.int32)
        slots = int(tile_ptr[-1].item())
        return (view(src, 4 * slots, torch.int32), view(row, 2 * slots, torch.int16),
                view(blk, 4 * (slots // 256), torch.int32), tile_ptr, row0, rows)

    @property
    def n(self) -> int:
        return self.graph.n

    def buckets(self):
        return pr_plan_buckets(self.handle)

    def run(self, d: float = 0.85, tol: float = 0.0, max_iter: int = 50, x0=None,
            record_events: bool = False, sum_trace: bool = True, stream=None, out=None):
        torch = _torch()
        dev = self.graph.row_ptr.device
        x = out if out is not None else torch.empty(self.n, dtype=torch.float32, device=dev)
        flags = 0
        if x0 is not None:
            x.copy_(torch.as_tensor(x0, dtype=torch.float32))
            flags |= PR_X0_GIVEN
        if record_events:
            flags |= PR_RECORD_EVENTS
        l1 = torch.full((max_iter,), float("nan"), dtype=torch.float32, device=dev)
        st = torch.full((max_iter,), float("nan"), dtype=torch.float32, device=dev) if sum_trace else None
        it = pr_run(self.handle, d, tol, max_iter, x, l1, st, flags, stream)
        return RunResult(x, it, l1[:it], None if st is None else st[:it])

    def iteration_ms(self) -> float:
        return pr_plan_iteration_ms(self.handle)

    def kernel_ms(self) -> tuple[float, int]:
        return pr_plan_kernel_ms(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            pr_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class SpmvPlan:
    """Row schedule of a CSR sparsity pattern (pr_spmv_plan_create), ready for
    y = A x with pr_spmv.  Keeps the pattern tensors and the plan's workspace
    alive for its lifetime (the plan borrows row_ptr and col_idx)."""

    def __init__(self, row_ptr, col_idx, n_cols: int, flags: int = 0, stream=None):
        self.row_ptr, self.col_idx = row_ptr, col_idx
        self.n_rows = int(row_ptr.numel() - 1)
        self.n_cols = int(n_cols)
        self.nnz = int(col_idx.numel())
        dev = row_ptr.device
        self.ws = _device_buffer(pr_spmv_workspace_bytes(self.n_rows, self.nnz), dev)
        scratch = _device_buffer(pr_spmv_scratch_bytes(self.n_rows, self.nnz), dev)
        self.handle = pr_spmv_plan_create(self.n_rows, self.n_cols, self.nnz, row_ptr, col_idx,
                                          self.ws, scratch, flags, stream)
        del scratch

    @classmethod
    def from_csr(cls, row_ptr, col_idx, n_cols: int, device="cuda", flags: int = 0):
        g = DeviceGraph.from_csr(row_ptr, col_idx, device)
        return cls(g.row_ptr, g.col_idx, n_cols, flags)

    def items(self) -> dict:
        return pr_spmv_plan_items(self.handle)

    def run(self, vals, x, out=None, stream=None):
        """y = A x (float64 device tensors; vals in the pattern's order)."""
        torch = _torch()
        y = out if out is not None else torch.empty(self.n_rows, dtype=torch.float64,
                                                    device=self.row_ptr.device)
        for t, n in ((vals, self.nnz), (x, self.n_cols), (y, self.n_rows)):
            if t.dtype != torch.float64 or t.numel() != n or not t.is_contiguous():
                raise ValueError("vals, x and y must be contiguous float64 of nnz, n_cols "
                                 "and n_rows entries")
        pr_spmv(self.handle, vals, x, y, stream)
        return y

    def close(self) -> None:
        if getattr(self, "handle", None):
            pr_spmv_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
