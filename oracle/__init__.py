"""PageRank oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, double-precision CPU implementation of the method (the C file
``pr_oracle.c``; its header cites the passages it follows), wrapped for numpy.
Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library in
``pagerank_power_iteration_amd``, and that library never imports it.

Parity status of each function (what pins it is in the CPU tests):

* ``transpose`` -- pinned: lexicographic sort of (v, u) pairs, brute force over
  every digraph on 3 and 4 vertices, transpose of a transpose, symmetric
  stencil, in-degree counts.
* ``pagerank`` -- pinned: dense linear solve of (I - dP) x = (1-d)/n on graphs
  of at most 11 vertices, closed forms (cycle, no edges, complete digraph,
  single vertex, both stars, chain), the unit sum after every pass, the
  dropped-dangling total S' = (1-d) + d (S - D) with its fixed point and the
  proportionality of the broken vector, and the contraction L1_{t+1} <= d L1_t.
  On the large synthetic graphs no page prints values, so beyond these
  properties the values there are the oracle's own.
* ``spmv`` -- pinned: exact integer products against a dense int64 matrix
  product (square and rectangular, so a transposed operand fails), the exact
  rational sum within the rounding bound of a k-term sum, identity and
  diagonal matrices, empty rows, and the closed form of the 27-point stencil
  operator (-1 per neighbour, 27 on the diagonal) applied to the ones vector.
* ``bfs`` -- pinned: unweighted shortest paths from scipy's csgraph routine on
  random directed graphs, brute-force levels from powers of the boolean
  adjacency matrix on every digraph of 3 vertices, closed forms (directed
  chain and its reverse, cycle, both stars, the 2-D grid's Manhattan distance
  with depth 2 (side - 1) + 1), unreachable vertices, and the edge count.
* ``wcc`` -- pinned: scipy's weak connected components (relabelled by their
  smallest member) on random directed graphs, the transitive closure of the
  symmetrised adjacency on every digraph of 3 vertices, closed forms (no
  edges, one cycle, disjoint cycles, a reversed chain, the grid), and
  invariance under reversing every edge.
* ``ranking`` / ``top_k`` -- sort by (-x, id).
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DROP_DANGLING = 1


def build(verbose: bool = False) -> str:
    """Compile liboracle.so in place: plain gcc, single-threaded, -O2."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-Wall", "-o",
           _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


@functools.lru_cache(maxsize=1)
def _lib() -> ctypes.CDLL:
    if not os.path.exists(_LIB):
        raise RuntimeError(f"{_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.pro_transpose.argtypes = [ctypes.c_int32, ctypes.c_int64, i32p, i32p, i32p, i32p]
    lib.pro_transpose.restype = ctypes.c_int
    lib.pro_pagerank.argtypes = [ctypes.c_int32, ctypes.c_int64, i32p, i32p, ctypes.c_double,
                                 ctypes.c_double, ctypes.c_int32, f64p, ctypes.c_uint32, f64p,
                                 f64p, f64p, f64p, i32p, f64p]
    lib.pro_pagerank.restype = ctypes.c_int
    lib.pro_spmv.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, i32p, i32p, f64p,
                             f64p, f64p, f64p]
    lib.pro_spmv.restype = ctypes.c_int
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.pro_bfs.argtypes = [ctypes.c_int32, ctypes.c_int64, i32p, i32p, ctypes.c_int32, i32p, i32p,
                            i64p, f64p]
    lib.pro_bfs.restype = ctypes.c_int
    lib.pro_wcc.argtypes = [ctypes.c_int32, ctypes.c_int64, i32p, i32p, i32p, i32p, f64p]
    lib.pro_wcc.restype = ctypes.c_int
    return lib


def _p(a: np.ndarray | None, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _csr(row_ptr, col_idx):
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if ci.size == 0:
        ci = np.zeros(1, dtype=np.int32)[:0]
    return rp, ci


_ERRORS = {-1: "bad argument", -2: "malformed CSR", -3: "out of memory"}


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def transpose(row_ptr, col_idx):
    """In-edge CSR (in_row_ptr int32[n+1], in_col_idx int32[m]) of an out-edge CSR."""
    rp, ci = _csr(row_ptr, col_idx)
    n, m = rp.size - 1, ci.size
    in_rp = np.empty(n + 1, dtype=np.int32)
    in_ci = np.empty(max(m, 1), dtype=np.int32)
    _check(_lib().pro_transpose(n, m, _p(rp, ctypes.c_int32), _p(ci, ctypes.c_int32),
                                _p(in_rp, ctypes.c_int32), _p(in_ci, ctypes.c_int32)),
           "transpose")
    return in_rp, in_ci[:m]


class Result:
    __slots__ = ("x", "iterations", "l1_trace", "sum_trace", "dmass_trace", "loop_seconds")

    def __init__(self, x, iterations, l1, s, dm, secs):
        self.x, self.iterations = x, iterations
        self.l1_trace, self.sum_trace, self.dmass_trace = l1, s, dm
        self.loop_seconds = secs


def pagerank(row_ptr, col_idx, d: float = 0.85, tol: float = 0.0, max_iter: int = 100,
             x0=None, drop_dangling: bool = False) -> Result:
    """Power iteration on an out-edge CSR; see pr_oracle.h for the contract."""
    rp, ci = _csr(row_ptr, col_idx)
    n, m = rp.size - 1, ci.size
    x = np.empty(n, dtype=np.float64)
    l1 = np.zeros(max_iter, dtype=np.float64)
    s = np.zeros(max_iter, dtype=np.float64)
    dm = np.zeros(max_iter, dtype=np.float64)
    it = np.zeros(1, dtype=np.int32)
    secs = np.zeros(1, dtype=np.float64)
    x0a = None if x0 is None else np.ascontiguousarray(x0, dtype=np.float64)
    if x0a is not None and x0a.shape != (n,):
        raise ValueError("x0 has the wrong length")
    rc = _lib().pro_pagerank(n, m, _p(rp, ctypes.c_int32), _p(ci, ctypes.c_int32), float(d),
                             float(tol), int(max_iter), _p(x0a, ctypes.c_double),
                             DROP_DANGLING if drop_dangling else 0, _p(x, ctypes.c_double),
                             _p(l1, ctypes.c_double), _p(s, ctypes.c_double),
                             _p(dm, ctypes.c_double), _p(it, ctypes.c_int32),
                             _p(secs, ctypes.c_double))
    _check(rc, "pagerank")
    t = int(it[0])
    return Result(x, t, l1[:t], s[:t], dm[:t], float(secs[0]))


def spmv(row_ptr, col_idx, vals, x, n_cols: int | None = None, timed: bool = False):
    """y = A x for the valued CSR matrix (row_ptr, col_idx, vals); float64.
    With timed=True returns (y, seconds of the product loop)."""
    rp, ci = _csr(row_ptr, col_idx)
    va = np.ascontiguousarray(vals, dtype=np.float64)
    xa = np.ascontiguousarray(x, dtype=np.float64)
    n_rows, nnz = rp.size - 1, ci.size
    n_cols = xa.size if n_cols is None else int(n_cols)
    if va.size != nnz or xa.size != n_cols:
        raise ValueError("vals / x have the wrong length")
    y = np.empty(max(n_rows, 1), dtype=np.float64)
    secs = np.zeros(1, dtype=np.float64)
    _check(_lib().pro_spmv(n_rows, n_cols, nnz, _p(rp, ctypes.c_int32), _p(ci, ctypes.c_int32),
                           _p(va, ctypes.c_double), _p(xa, ctypes.c_double),
                           _p(y, ctypes.c_double), _p(secs, ctypes.c_double)), "spmv")
    y = y[:n_rows]
    return (y, float(secs[0])) if timed else y


class BfsResult:
    __slots__ = ("level", "depth", "edges_scanned", "loop_seconds")

    def __init__(self, level, depth, edges, secs):
        self.level, self.depth, self.edges_scanned, self.loop_seconds = level, depth, edges, secs


def bfs(row_ptr, col_idx, source: int) -> BfsResult:
    """Breadth-first levels from `source` over the out-edges (-1: unreachable)."""
    rp, ci = _csr(row_ptr, col_idx)
    n, m = rp.size - 1, ci.size
    level = np.empty(max(n, 1), dtype=np.int32)
    depth = np.zeros(1, dtype=np.int32)
    edges = np.zeros(1, dtype=np.int64)
    secs = np.zeros(1, dtype=np.float64)
    _check(_lib().pro_bfs(n, m, _p(rp, ctypes.c_int32), _p(ci, ctypes.c_int32), int(source),
                          _p(level, ctypes.c_int32), _p(depth, ctypes.c_int32),
                          _p(edges, ctypes.c_int64), _p(secs, ctypes.c_double)), "bfs")
    return BfsResult(level[:n], int(depth[0]), int(edges[0]), float(secs[0]))


def wcc(row_ptr, col_idx, timed: bool = False):
    """Weakly connected components: label[v] = smallest id in v's component.
    Returns (label, n_components), plus the search's seconds with timed=True."""
    rp, ci = _csr(row_ptr, col_idx)
    n, m = rp.size - 1, ci.size
    label = np.empty(max(n, 1), dtype=np.int32)
    comps = np.zeros(1, dtype=np.int32)
    secs = np.zeros(1, dtype=np.float64)
    _check(_lib().pro_wcc(n, m, _p(rp, ctypes.c_int32), _p(ci, ctypes.c_int32),
                          _p(label, ctypes.c_int32), _p(comps, ctypes.c_int32),
                          _p(secs, ctypes.c_double)), "wcc")
    out = (label[:n], int(comps[0]))
    return out + (float(secs[0]),) if timed else out


def ranking(x) -> np.ndarray:
    """Vertex ids by decreasing rank, ties by increasing id."""
    x = np.asarray(x)
    return np.lexsort((np.arange(x.size), -x.astype(np.float64)))


def top_k(x, k: int = 20) -> np.ndarray:
    return ranking(x)[:k]
