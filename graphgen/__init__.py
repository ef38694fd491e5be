"""Seeded synthetic graph inputs (out-edge CSR, int32), shared by every test
and by the benchmark.

Holds no PageRank arithmetic and no transpose: it only makes graphs.  The
large generators are C (``graphgen.c``, OpenMP); small named graphs are built
here with numpy.

Workloads (the shapes of the pages' graphs; none of their data):

* ``citation``   -- 28,042 papers, 2,204 of which cite nothing ("100 Days of
  GPU" Day 40, the real citation graph's counts); the others cite a
  geometric number of papers with mean 12, each target drawn with probability
  proportional to in-degree + 1.  Stands in for the page's citation graph,
  which is not available here.
* ``stencil100`` -- 27-point stencil on a 100^3 grid ("A Pedagogical
  Introduction to Porting a Conjugate Gradient Solver to CUDA", the HPCCG
  problem's 100^3 size): n = 10^6, m = 298^3 - 10^6 = 25,463,592.
* ``rmatS``      -- R-MAT scale S, edge factor 32, (a, b, c, d) =
  (0.57, 0.19, 0.19, 0.05), seed S, self-loops and duplicates removed
  ("gpu-graph-study", scale study over 2^18 .. 2^23 vertices).

Every CSR has rows sorted by target with no duplicates and no self-loops,
except graphs built with ``from_edges(..., dedup=False)``.

Valued matrices (the sparse product's inputs, class ``Matrix``):

* ``stencil_matrix`` -- the 27-point stencil with its diagonal (the HPCCG
  operator's shape in the conjugate-gradient porting article; 100^3 gives
  26,463,592 stored entries).  The article does not print the values; ``values="operator"`` takes -1 for every
  neighbour and 27 on the diagonal (diagonally dominant, and A times the
  ones vector is 1 on interior rows), ``values="random"`` draws each entry
  uniformly from [-1, 1).
* ``matrix_from_lengths`` -- given row lengths, seeded uniform columns and
  values; used for rows that straddle every length class of the product.
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "graphgen.c")
_LIB = os.path.join(_HERE, "libgraphgen.so")

RMAT_ABC = (0.57, 0.19, 0.19)


def build(verbose: bool = False) -> str:
    """Compile libgraphgen.so in place (gcc, OpenMP)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
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
    p32 = ctypes.POINTER(ctypes.POINTER(ctypes.c_int32))
    pm = ctypes.POINTER(ctypes.c_int64)
    lib.gg_rmat.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                            ctypes.c_double, ctypes.c_uint64, p32, p32, pm]
    lib.gg_stencil27.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, p32, p32, pm]
    lib.gg_citation.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_uint64,
                                p32, p32, pm]
    for f in (lib.gg_rmat, lib.gg_stencil27, lib.gg_citation):
        f.restype = ctypes.c_int
    i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.gg_rmat_edges.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, i32p, i32p]
    lib.gg_relabel.argtypes = [ctypes.c_int32, i32p, i32p, i32p, p32, p32, pm]
    lib.gg_edit.argtypes = [ctypes.c_int32, i32p, i32p, ctypes.c_int64, i64p, ctypes.c_int64,
                            i32p, i32p, p32, p32, pm]
    for f in (lib.gg_rmat_edges, lib.gg_relabel, lib.gg_edit):
        f.restype = ctypes.c_int
    lib.gg_free.argtypes = [ctypes.c_void_p]
    lib.gg_free.restype = None
    lib.gg_draw_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.gg_draw_u64.restype = ctypes.c_uint64
    lib.gg_num_threads.restype = ctypes.c_int
    return lib


class Graph:
    """Out-edge CSR: ``row_ptr`` int32[n+1], ``col_idx`` int32[m]."""

    __slots__ = ("name", "n", "row_ptr", "col_idx")

    def __init__(self, name: str, row_ptr: np.ndarray, col_idx: np.ndarray):
        self.name = name
        self.row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        self.col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
        self.n = int(self.row_ptr.shape[0] - 1)

    @property
    def m(self) -> int:
        return int(self.col_idx.shape[0])

    def out_degree(self) -> np.ndarray:
        return np.diff(self.row_ptr.astype(np.int64))

    def n_dangling(self) -> int:
        return int(np.count_nonzero(self.out_degree() == 0))

    def edges(self):
        src = np.repeat(np.arange(self.n, dtype=np.int32), self.out_degree())
        return src, self.col_idx.copy()

    def __repr__(self) -> str:
        return f"Graph({self.name!r}, n={self.n}, m={self.m})"


def _take(name: str, rc: int, rp, ci, m, n: int) -> Graph:
    lib = _lib()
    if rc != 0:
        raise ValueError(f"graph generator {name} failed with code {rc}")
    try:
        row_ptr = np.ctypeslib.as_array(rp, shape=(n + 1,)).copy()
        col_idx = (np.ctypeslib.as_array(ci, shape=(m.value,)).copy() if m.value > 0
                   else np.zeros(0, dtype=np.int32))
    finally:
        lib.gg_free(ctypes.cast(rp, ctypes.c_void_p))
        lib.gg_free(ctypes.cast(ci, ctypes.c_void_p))
    return Graph(name, row_ptr, col_idx)


def rmat(scale: int, edge_factor: int = 32, abc=RMAT_ABC, seed: int | None = None) -> Graph:
    """R-MAT graph with 2**scale vertices and edge_factor * 2**scale draws."""
    seed = scale if seed is None else seed
    rp, ci, m = (ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)(),
                 ctypes.c_int64())
    rc = _lib().gg_rmat(scale, edge_factor << scale, abc[0], abc[1], abc[2], seed,
                        ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(m))
    return _take(f"rmat{scale}", rc, rp, ci, m, 1 << scale)


def stencil27(nx: int, ny: int | None = None, nz: int | None = None) -> Graph:
    ny = nx if ny is None else ny
    nz = nx if nz is None else nz
    rp, ci, m = (ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)(),
                 ctypes.c_int64())
    rc = _lib().gg_stencil27(nx, ny, nz, ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(m))
    return _take(f"stencil{nx}x{ny}x{nz}", rc, rp, ci, m, nx * ny * nz)


def citation(n: int = 28042, n_dangling: int = 2204, mean_outdeg: float = 12.0,
             seed: int = 40) -> Graph:
    rp, ci, m = (ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)(),
                 ctypes.c_int64())
    rc = _lib().gg_citation(n, n_dangling, mean_outdeg, seed, ctypes.byref(rp),
                            ctypes.byref(ci), ctypes.byref(m))
    return _take("citation", rc, rp, ci, m, n)


# ----------------------------------------------------------------- small graphs

def splitmix_u64(seed: int, counters: np.ndarray) -> np.ndarray:
    """Vectorised counter-based SplitMix64 draws (same stream as graphgen.c)."""
    with np.errstate(over="ignore"):
        def mix(z):
            z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
            z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
            return z ^ (z >> np.uint64(31))
        key = mix(np.array([seed], dtype=np.uint64))[0]
        k = np.asarray(counters, dtype=np.uint64)
        return mix(key + (k + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15))


def from_edges(n: int, src, dst, dedup: bool = True, drop_self: bool = True,
               name: str = "edges") -> Graph:
    """Out-edge CSR from an edge list; rows sorted by target."""
    src = np.asarray(src, dtype=np.int64).ravel()
    dst = np.asarray(dst, dtype=np.int64).ravel()
    if src.shape != dst.shape:
        raise ValueError("src and dst differ in length")
    if src.size and (src.min() < 0 or src.max() >= n or dst.min() < 0 or dst.max() >= n):
        raise ValueError("vertex id out of range")
    if drop_self:
        keep = src != dst
        src, dst = src[keep], dst[keep]
    order = np.lexsort((dst, src))
    src, dst = src[order], dst[order]
    if dedup and src.size:
        keep = np.ones(src.size, dtype=bool)
        keep[1:] = (src[1:] != src[:-1]) | (dst[1:] != dst[:-1])
        src, dst = src[keep], dst[keep]
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(np.bincount(src, minlength=n))
    return Graph(name, row_ptr.astype(np.int32), dst.astype(np.int32))


def random_graph(n: int, m_draws: int, seed: int, name: str | None = None,
                 dedup: bool = True, drop_self: bool = True) -> Graph:
    """Uniform random digraph from m_draws seeded (u, v) draws."""
    k = np.arange(2 * m_draws, dtype=np.uint64)
    r = splitmix_u64(seed, k) % np.uint64(max(n, 1))
    src, dst = r[0::2].astype(np.int64), r[1::2].astype(np.int64)
    return from_edges(n, src, dst, dedup=dedup, drop_self=drop_self,
                      name=name or f"random{n}_{m_draws}_{seed}")


def empty(n: int) -> Graph:
    return Graph(f"empty{n}", np.zeros(n + 1, dtype=np.int32), np.zeros(0, dtype=np.int32))


def cycle(n: int) -> Graph:
    u = np.arange(n)
    return from_edges(n, u, (u + 1) % n, name=f"cycle{n}")


def chain(n: int) -> Graph:
    u = np.arange(n - 1)
    return from_edges(n, u, u + 1, name=f"chain{n}")


def complete(n: int) -> Graph:
    u, v = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    return from_edges(n, u.ravel(), v.ravel(), name=f"complete{n}")


def star(n: int, inward: bool = True) -> Graph:
    """Hub 0 and n-1 leaves; inward: every leaf points at the hub."""
    leaves = np.arange(1, n)
    hub = np.zeros(n - 1, dtype=np.int64)
    if inward:
        return from_edges(n, leaves, hub, name=f"star{n}_in")
    return from_edges(n, hub, leaves, name=f"star{n}_out")


def grid2d(nx: int, ny: int | None = None) -> Graph:
    """4-neighbour grid, both directions of every link; vertex id = x + nx*y.
    1024 x 1024 is the high-diameter graph of the graph study's traversal
    tables (2^20 vertices, 4,190,208 directed edges, BFS depth 2046 from a
    corner)."""
    ny = nx if ny is None else ny
    x, y = np.meshgrid(np.arange(nx, dtype=np.int64), np.arange(ny, dtype=np.int64),
                       indexing="xy")
    x, y = x.ravel(), y.ravel()
    v = x + nx * y
    src, dst = [], []
    for dx, dy in ((1, 0), (-1, 0), (0, 1), (0, -1)):
        ok = (x + dx >= 0) & (x + dx < nx) & (y + dy >= 0) & (y + dy < ny)
        src.append(v[ok])
        dst.append(v[ok] + dx + nx * dy)
    return from_edges(nx * ny, np.concatenate(src), np.concatenate(dst),
                      name=f"grid{nx}x{ny}")


def tiny() -> Graph:
    """6 vertices, 9 edges, vertex 5 dangling."""
    src = [0, 0, 1, 1, 2, 3, 3, 4, 4]
    dst = [1, 2, 2, 3, 0, 4, 5, 0, 5]
    return from_edges(6, src, dst, name="tiny")


def single() -> Graph:
    return Graph("single", np.zeros(2, dtype=np.int32), np.zeros(0, dtype=np.int32))


def two_out(n: int, seed: int, name: str) -> Graph:
    """Every vertex has exactly two distinct out-neighbours other than itself."""
    off = splitmix_u64(seed, np.arange(2 * n, dtype=np.uint64))
    a = 1 + (off[0::2] % np.uint64(n - 1)).astype(np.int64)
    b = 1 + (off[1::2] % np.uint64(n - 2)).astype(np.int64)
    b = np.where(b >= a, b + 1, b)  # distinct from a, still in 1..n-1
    u = np.arange(n, dtype=np.int64)
    src = np.concatenate([u, u])
    dst = np.concatenate([(u + a) % n, (u + b) % n])
    return from_edges(n, src, dst, name=name)


def nodangling(n: int = 4096, seed: int = 7) -> Graph:
    return two_out(n, seed, "nodangling")


def dangling(n: int = 4096, n_dangling: int = 400, seed: int = 7) -> Graph:
    """``nodangling`` with the out-edges of a seeded sample of vertices removed."""
    g = two_out(n, seed, "dangling")
    keys = splitmix_u64(seed + 1, np.arange(n, dtype=np.uint64))
    drop = np.argsort(keys, kind="stable")[:n_dangling]
    src, dst = g.edges()
    keep = ~np.isin(src, drop)
    return from_edges(n, src[keep], dst[keep], name="dangling")


# --------------------------------------------------------------- valued matrices

class Matrix:
    """Valued CSR: ``row_ptr`` int32[n_rows+1], ``col_idx`` int32[nnz],
    ``vals`` float64[nnz], columns in [0, n_cols)."""

    __slots__ = ("name", "n_rows", "n_cols", "row_ptr", "col_idx", "vals")

    def __init__(self, name: str, row_ptr, col_idx, vals, n_cols: int):
        self.name = name
        self.row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        self.col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
        self.vals = np.ascontiguousarray(vals, dtype=np.float64)
        self.n_rows = int(self.row_ptr.shape[0] - 1)
        self.n_cols = int(n_cols)

    @property
    def nnz(self) -> int:
        return int(self.col_idx.shape[0])

    def row_lengths(self) -> np.ndarray:
        return np.diff(self.row_ptr.astype(np.int64))

    def __repr__(self) -> str:
        return f"Matrix({self.name!r}, {self.n_rows}x{self.n_cols}, nnz={self.nnz})"


def uniform(n: int, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """n seeded draws, uniform in [lo, hi), float64 (53-bit mantissas)."""
    u = (splitmix_u64(seed, np.arange(n, dtype=np.uint64)) >> np.uint64(11)).astype(np.float64)
    return lo + (hi - lo) * (u * (1.0 / 9007199254740992.0))


def small_ints(n: int, seed: int, bound: int = 8) -> np.ndarray:
    """n seeded integers in [-bound, bound], as float64."""
    r = splitmix_u64(seed, np.arange(n, dtype=np.uint64)) % np.uint64(2 * bound + 1)
    return r.astype(np.float64) - bound


def stencil_matrix(nx: int, ny: int | None = None, nz: int | None = None,
                   values: str = "operator", seed: int = 1) -> Matrix:
    """27-point stencil on an nx*ny*nz grid with the diagonal stored in place
    (columns ascending in every row)."""
    g = stencil27(nx, ny, nz)
    n = g.n
    deg = g.out_degree()
    rows = np.repeat(np.arange(n, dtype=np.int64), deg)
    after = (g.col_idx > rows).astype(np.int64)
    e = np.arange(g.m, dtype=np.int64)
    row_ptr = g.row_ptr.astype(np.int64) + np.arange(n + 1, dtype=np.int64)
    col = np.empty(g.m + n, dtype=np.int32)
    is_diag = np.ones(g.m + n, dtype=bool)
    pos = e + rows + after
    col[pos] = g.col_idx
    is_diag[pos] = False
    col[is_diag] = np.arange(n, dtype=np.int32)
    if values == "operator":
        vals = np.where(is_diag, 27.0, -1.0)
    elif values == "random":
        vals = uniform(g.m + n, seed)
    else:
        raise ValueError(values)
    return Matrix(f"stencil_matrix{g.name[7:]}_{values}", row_ptr, col, vals, n)


def matrix_from_lengths(lengths, n_cols: int, seed: int, int_values: bool = False,
                        name: str | None = None) -> Matrix:
    """Rows of the given lengths; columns uniform in [0, n_cols) (repeats
    allowed, stored order unsorted), values uniform in [-1, 1) or small
    integers."""
    lengths = np.asarray(lengths, dtype=np.int64)
    row_ptr = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=row_ptr[1:])
    nnz = int(row_ptr[-1])
    col = (splitmix_u64(seed, np.arange(nnz, dtype=np.uint64)) % np.uint64(max(n_cols, 1)))
    vals = small_ints(nnz, seed + 1) if int_values else uniform(nnz, seed + 1)
    return Matrix(name or f"rows{lengths.size}_{nnz}_{seed}", row_ptr, col.astype(np.int32),
                  vals, n_cols)


def matrix_of_graph(g: Graph, seed: int) -> Matrix:
    """The graph's out-edge CSR with seeded uniform values in [-1, 1)."""
    return Matrix(f"{g.name}_valued", g.row_ptr, g.col_idx, uniform(g.m, seed), g.n)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def relabel(g: Graph, seed: int, name: str | None = None) -> Graph:
    """The same graph with its vertex ids shuffled by a seeded permutation:
    vertex v becomes perm[v], where perm sorts the vertices by their
    SplitMix64 draw (ties by id).  Kills whatever locality the generator's
    ids carry (R-MAT's hot vertices sit at ids with few one bits)."""
    perm = relabel_permutation(g.n, seed)
    rp, ci, m = (ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)(),
                 ctypes.c_int64())
    rc = _lib().gg_relabel(g.n, _i32p(g.row_ptr), _i32p(g.col_idx), _i32p(perm),
                           ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(m))
    return _take(name or f"{g.name}_relabelled", rc, rp, ci, m, g.n)


def relabel_permutation(n: int, seed: int) -> np.ndarray:
    keys = splitmix_u64(seed, np.arange(n, dtype=np.uint64))
    order = np.lexsort((np.arange(n), keys))
    perm = np.empty(n, dtype=np.int32)
    perm[order] = np.arange(n, dtype=np.int32)
    return perm


def edge_batch(g: Graph, n_delete: int, n_insert: int, seed: int):
    """A seeded batch of edge deletions and insertions: the indices (into
    g.col_idx, ascending) of n_delete distinct existing edges, drawn
    uniformly, and n_insert new (u, v) draws -- R-MAT draws with the
    workload's parameters when n is a power of two, uniform pairs otherwise
    (self-loops and edges already present are dropped when applied)."""
    m = g.m
    n_delete = min(n_delete, m)
    k, picked = 0, np.zeros(0, dtype=np.int64)
    while picked.size < n_delete:
        want = 2 * (n_delete - picked.size) + 16
        cand = (splitmix_u64(seed, np.arange(k, k + want, dtype=np.uint64)) %
                np.uint64(m)).astype(np.int64)
        k += want
        _, first = np.unique(np.concatenate([picked, cand]), return_index=True)
        merged = np.concatenate([picked, cand])[np.sort(first)]
        picked = merged[:n_delete]
    dele = np.sort(picked)
    scale = g.n.bit_length() - 1
    u = np.empty(n_insert, dtype=np.int32)
    v = np.empty(n_insert, dtype=np.int32)
    if g.n == 1 << scale and scale >= 1:
        rc = _lib().gg_rmat_edges(scale, RMAT_ABC[0], RMAT_ABC[1], RMAT_ABC[2], seed + 1, 0,
                                  n_insert, _i32p(u), _i32p(v))
        if rc != 0:
            raise ValueError(f"gg_rmat_edges failed with code {rc}")
    else:
        r = splitmix_u64(seed + 1, np.arange(2 * n_insert, dtype=np.uint64)) % np.uint64(g.n)
        u[:], v[:] = r[:n_insert], r[n_insert:]
    return dele, u, v


def apply_batch(g: Graph, dele: np.ndarray, ins_u: np.ndarray, ins_v: np.ndarray,
                name: str | None = None) -> Graph:
    """g with the edges at indices `dele` (ascending) removed and the edges
    (ins_u[i], ins_v[i]) added (no self-loops, no duplicates)."""
    dele = np.ascontiguousarray(dele, dtype=np.int64)
    ins_u = np.ascontiguousarray(ins_u, dtype=np.int32)
    ins_v = np.ascontiguousarray(ins_v, dtype=np.int32)
    rp, ci, m = (ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)(),
                 ctypes.c_int64())
    rc = _lib().gg_edit(g.n, _i32p(g.row_ptr), _i32p(g.col_idx), dele.size,
                        dele.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ins_u.size,
                        _i32p(ins_u), _i32p(ins_v), ctypes.byref(rp), ctypes.byref(ci),
                        ctypes.byref(m))
    return _take(name or f"{g.name}_edited", rc, rp, ci, m, g.n)


RELABEL_SEED = 2323


def workload(name: str) -> Graph:
    """The named benchmark workloads ("rmat23r": R-MAT 23 with its vertex ids
    shuffled by a seeded permutation)."""
    if name.endswith("r") and name.startswith("rmat"):
        return relabel(rmat(int(name[4:-1])), RELABEL_SEED, name=name)
    if name == "citation":
        return citation()
    if name == "stencil100":
        return stencil27(100)
    if name.startswith("rmat"):
        return rmat(int(name[4:]))
    if name == "grid1024":
        return grid2d(1024)
    raise KeyError(name)


WORKLOADS = ("citation", "stencil100", "rmat18", "rmat21", "rmat23")
