"""ctypes binding of libpr.so (include/pr.h), one Python function per C entry
point with the same name.  Argument marshalling only: tensors become device
pointers, the stream defaults to torch's current stream, and a negative
status becomes a PrError carrying pr_last_error().  No computation happens
here, and there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libpr.so")
HEADER = os.path.join(ROOT, "include", "pr.h")

PR_OK = 0
PR_ERR_ARG = -1
PR_ERR_WORKSPACE = -2
PR_ERR_GRAPH = -3
PR_ERR_HIP = -4

PR_VALIDATE = 0x1
PR_PLAN_BUCKETED = 0x2
PR_X0_GIVEN = 0x1
PR_RECORD_EVENTS = 0x2
PR_NOALLOC_SCRATCH_BYTES = 128 << 20


class PrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


_c = ctypes
_vp = _c.c_void_p
_SIGNATURES = {
    "pr_transpose_workspace_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_transpose": (_c.c_int, [_c.c_int32, _c.c_int64, _vp, _vp, _vp, _vp, _vp, _c.c_size_t,
                                _c.c_uint32, _vp]),
    "pr_transpose_noalloc": (_c.c_int, [_c.c_int32, _c.c_int64, _vp, _vp, _vp, _vp, _c.c_uint32,
                                        _vp]),
    "pr_plan_workspace_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_plan_scratch_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_plan_create": (_c.c_int, [_c.POINTER(_vp), _c.c_int32, _c.c_int64, _vp, _vp, _vp,
                                  _c.c_size_t, _vp, _c.c_size_t, _c.c_uint32, _vp]),
    "pr_plan_destroy": (_c.c_int, [_vp]),
    "pr_run": (_c.c_int, [_vp, _c.c_double, _c.c_double, _c.c_int32, _vp, _vp, _vp,
                          _c.POINTER(_c.c_int32), _c.c_uint32, _vp]),
    "pr_plan_iteration_ms": (_c.c_int, [_vp, _c.POINTER(_c.c_float)]),
    "pr_plan_kernel_ms": (_c.c_int, [_vp, _c.POINTER(_c.c_float), _c.POINTER(_c.c_int32)]),
    "pr_plan_num_buckets": (_c.c_int, []),
    "pr_plan_buckets": (_c.c_int, [_vp, _c.POINTER(_c.c_int32), _c.POINTER(_c.c_int32),
                                   _c.POINTER(_c.c_int64)]),
    "pr_plan_layout": (_c.c_int, [_vp, _c.POINTER(_vp), _c.POINTER(_vp), _c.POINTER(_vp)]),
    "pr_plan_tiles": (_c.c_int, [_vp, _c.POINTER(_vp), _c.POINTER(_vp), _c.POINTER(_vp),
                                 _c.POINTER(_vp), _c.POINTER(_c.c_int32), _vp, _vp]),
    "pr_spmv_workspace_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_spmv_scratch_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_spmv_plan_create": (_c.c_int, [_c.POINTER(_vp), _c.c_int32, _c.c_int32, _c.c_int64, _vp,
                                       _vp, _vp, _c.c_size_t, _vp, _c.c_size_t, _c.c_uint32,
                                       _vp]),
    "pr_spmv_plan_destroy": (_c.c_int, [_vp]),
    "pr_spmv": (_c.c_int, [_vp, _vp, _vp, _vp, _vp]),
    "pr_spmv_plan_items": (_c.c_int, [_vp, _c.POINTER(_c.c_int32)]),
    "pr_bfs_workspace_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_bfs": (_c.c_int, [_c.c_int32, _c.c_int64, _vp, _vp, _vp, _vp, _c.c_int32, _vp,
                          _c.POINTER(_c.c_int32), _c.POINTER(_c.c_int64), _vp, _c.c_size_t,
                          _c.c_uint32, _vp]),
    "pr_wcc_workspace_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64]),
    "pr_wcc": (_c.c_int, [_c.c_int32, _c.c_int64, _vp, _vp, _vp, _vp, _vp, _c.POINTER(_c.c_int32), _vp,
                          _c.c_size_t, _c.c_uint32, _vp]),
    "pr_status_string": (_c.c_char_p, [_c.c_int]),
    "pr_last_error": (_c.c_char_p, []),
}


def header_functions() -> list[str]:
    """Names of the functions include/pr.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pr_[a-z_0-9]+)\s*\(", text)))


@functools.lru_cache(maxsize=1)
def lib() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: the HIP library is not built (run __graft_entry__.build())")
    so = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


def _check(status: int) -> None:
    if status != PR_OK:
        msg = lib().pr_last_error().decode(errors="replace")
        raise PrError(status, f"{lib().pr_status_string(status).decode()}: {msg}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------ entry points

def pr_transpose_workspace_bytes(n: int, nnz: int) -> int:
    return int(lib().pr_transpose_workspace_bytes(n, nnz))


def pr_transpose(n, nnz, out_row_ptr, out_col_idx, in_row_ptr, in_col_idx, ws, flags=0,
                 stream=None) -> None:
    _check(lib().pr_transpose(n, nnz, _ptr(out_row_ptr), _ptr(out_col_idx), _ptr(in_row_ptr),
                              _ptr(in_col_idx), _ptr(ws), _nbytes(ws), flags, _stream(stream)))


def pr_transpose_noalloc(n, nnz, out_row_ptr, out_col_idx, in_row_ptr, in_col_idx, flags=0,
                         stream=None) -> None:
    _check(lib().pr_transpose_noalloc(n, nnz, _ptr(out_row_ptr), _ptr(out_col_idx),
                                      _ptr(in_row_ptr), _ptr(in_col_idx), flags,
                                      _stream(stream)))


def pr_plan_workspace_bytes(n: int, nnz: int) -> int:
    return int(lib().pr_plan_workspace_bytes(n, nnz))


def pr_plan_scratch_bytes(n: int, nnz: int) -> int:
    return int(lib().pr_plan_scratch_bytes(n, nnz))


def pr_plan_create(n, nnz, out_row_ptr, out_col_idx, ws, scratch, flags=0, stream=None) -> int:
    h = _vp()
    _check(lib().pr_plan_create(_c.byref(h), n, nnz, _ptr(out_row_ptr), _ptr(out_col_idx),
                                _ptr(ws), _nbytes(ws), _ptr(scratch), _nbytes(scratch), flags,
                                _stream(stream)))
    return h.value


def pr_plan_layout(plan) -> tuple[int, int, int | None]:
    """Device addresses of the plan's in_row_ptr, in_col_idx and new_id."""
    rp, ci, nid = _vp(), _vp(), _vp()
    _check(lib().pr_plan_layout(plan, _c.byref(rp), _c.byref(ci), _c.byref(nid)))
    return rp.value, ci.value, nid.value


def pr_plan_tiles(plan):
    """Device addresses of the tiled plan's tile_src, tile_row, tile_block and
    tile_ptr, and each tile's first plan id and row count (numpy arrays)."""
    import numpy as np
    src, row, blk, ptr = _vp(), _vp(), _vp(), _vp()
    nt = _c.c_int32(0)
    _check(lib().pr_plan_tiles(plan, _c.byref(src), _c.byref(row), _c.byref(blk), _c.byref(ptr),
                               _c.byref(nt), None, None))
    row0 = np.zeros(nt.value, dtype=np.int32)
    rows = np.zeros(nt.value, dtype=np.int32)
    _check(lib().pr_plan_tiles(plan, None, None, None, None, None, row0.ctypes.data,
                               rows.ctypes.data))
    return src.value, row.value, blk.value, ptr.value, nt.value, row0, rows


def pr_plan_destroy(plan: int | None) -> None:
    _check(lib().pr_plan_destroy(plan))


def pr_run(plan, d, tol, max_iter, x, l1_trace, sum_trace=None, flags=0, stream=None) -> int:
    it = _c.c_int32(0)
    _check(lib().pr_run(plan, float(d), float(tol), int(max_iter), _ptr(x), _ptr(l1_trace),
                        _ptr(sum_trace), _c.byref(it), flags, _stream(stream)))
    return int(it.value)


def pr_plan_iteration_ms(plan) -> float:
    ms = _c.c_float(0.0)
    _check(lib().pr_plan_iteration_ms(plan, _c.byref(ms)))
    return float(ms.value)


def pr_plan_kernel_ms(plan) -> tuple[float, int]:
    """(mean duration in ms of the main gather kernel's launches -- k_tile, or k_iterate
    for a bucketed plan -- and the number of launches averaged)."""
    ms = _c.c_float(0.0)
    k = _c.c_int32(0)
    _check(lib().pr_plan_kernel_ms(plan, _c.byref(ms), _c.byref(k)))
    return float(ms.value), int(k.value)


def pr_plan_num_buckets() -> int:
    return int(lib().pr_plan_num_buckets())


def pr_plan_buckets(plan) -> list[dict]:
    nb = pr_plan_num_buckets()
    mins = (_c.c_int32 * nb)()
    rows = (_c.c_int32 * nb)()
    edges = (_c.c_int64 * nb)()
    _check(lib().pr_plan_buckets(plan, mins, rows, edges))
    return [{"min_len": mins[b], "rows": rows[b], "edges": edges[b]} for b in range(nb)]


def pr_spmv_workspace_bytes(n_rows: int, nnz: int) -> int:
    return int(lib().pr_spmv_workspace_bytes(n_rows, nnz))


def pr_spmv_scratch_bytes(n_rows: int, nnz: int) -> int:
    return int(lib().pr_spmv_scratch_bytes(n_rows, nnz))


def pr_spmv_plan_create(n_rows, n_cols, nnz, row_ptr, col_idx, ws, scratch, flags=0,
                        stream=None) -> int:
    h = _vp()
    _check(lib().pr_spmv_plan_create(_c.byref(h), n_rows, n_cols, nnz, _ptr(row_ptr),
                                     _ptr(col_idx), _ptr(ws), _nbytes(ws), _ptr(scratch),
                                     _nbytes(scratch), flags, _stream(stream)))
    return h.value


def pr_spmv_plan_destroy(plan: int | None) -> None:
    _check(lib().pr_spmv_plan_destroy(plan))


def pr_spmv(plan, vals, x, y, stream=None) -> None:
    _check(lib().pr_spmv(plan, _ptr(vals), _ptr(x), _ptr(y), _stream(stream)))


def pr_spmv_plan_items(plan) -> dict:
    """Streamed blocks, 65..1024-entry rows, longer rows and their chunks."""
    c = (_c.c_int32 * 4)()
    _check(lib().pr_spmv_plan_items(plan, c))
    return {"blocks": c[0], "medium_rows": c[1], "long_rows": c[2], "chunks": c[3]}


def pr_bfs_workspace_bytes(n: int, nnz: int) -> int:
    return int(lib().pr_bfs_workspace_bytes(n, nnz))


def pr_bfs(n, nnz, row_ptr, col_idx, source, level, ws, in_row_ptr=None, in_col_idx=None,
           flags=0, stream=None) -> tuple[int, int]:
    """Breadth-first levels into `level`; returns (depth, edges scanned).
    Bottom-up levels need the in-edge CSR.  Synchronizes the stream."""
    depth = _c.c_int32(0)
    scanned = _c.c_int64(0)
    _check(lib().pr_bfs(n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(in_row_ptr),
                        _ptr(in_col_idx), int(source), _ptr(level), _c.byref(depth),
                        _c.byref(scanned), _ptr(ws), _nbytes(ws), flags, _stream(stream)))
    return depth.value, scanned.value


def pr_wcc_workspace_bytes(n: int, nnz: int) -> int:
    return int(lib().pr_wcc_workspace_bytes(n, nnz))


def pr_wcc(n, nnz, row_ptr, col_idx, label, ws, in_row_ptr=None, in_col_idx=None, flags=0,
           stream=None, count_components: bool = True) -> int | None:
    """Weak-component labels into `label`; returns the number of components
    (which synchronizes the stream) or None with count_components=False."""
    comps = _c.c_int32(0)
    _check(lib().pr_wcc(n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(in_row_ptr),
                        _ptr(in_col_idx), _ptr(label),
                        _c.byref(comps) if count_components else None, _ptr(ws), _nbytes(ws),
                        flags, _stream(stream)))
    return comps.value if count_components else None


def pr_status_string(status: int) -> str:
    return lib().pr_status_string(status).decode()


def pr_last_error() -> str:
    return lib().pr_last_error().decode(errors="replace")
