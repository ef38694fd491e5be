"""Pins of the breadth-first search and weakly-connected-components oracle
("gpu-graph-study", sections "Traversal (BFS / WCC)" and "Traversal T4 --
degree-bucketed BFS / WCC") against things other than itself: scipy's
csgraph routines, brute force over every digraph on 3 vertices, closed forms
(chains, cycles, stars, the 2-D grid whose corner search is 2046 levels deep
at 1024 x 1024, as the page's grid row states), and invariants."""
import itertools

import numpy as np
import pytest
import scipy.sparse as sp
from scipy.sparse import csgraph

import graphgen
import oracle
from tests import _pins


def _scipy_matrix(g):
    data = np.ones(g.m, dtype=np.float64)
    return sp.csr_matrix((data, g.col_idx, g.row_ptr), shape=(g.n, g.n))


def _min_id_labels(comp: np.ndarray) -> np.ndarray:
    """Relabel any component numbering by each component's smallest member."""
    first = np.full(comp.max() + 1, np.iinfo(np.int64).max, dtype=np.int64)
    np.minimum.at(first, comp, np.arange(comp.size))
    return first[comp]


RANDOM = [graphgen.random_graph(50, 60, 1), graphgen.random_graph(500, 700, 2),
          graphgen.random_graph(2000, 2500, 3), graphgen.random_graph(2000, 9000, 4),
          graphgen.random_graph(300, 2000, 5, dedup=False, drop_self=False),
          graphgen.rmat(10), graphgen.tiny(), graphgen.dangling(512, 60)]


# ---------------------------------------------------------------------- BFS

@pytest.mark.parametrize("g", RANDOM, ids=lambda g: g.name)
def test_bfs_matches_scipy_shortest_paths(g):
    M = _scipy_matrix(g)
    for s in (0, 1, g.n // 2, g.n - 1):
        r = oracle.bfs(g.row_ptr, g.col_idx, s)
        dist = csgraph.shortest_path(M, directed=True, unweighted=True, indices=s)
        ref = np.where(np.isinf(dist), -1, dist).astype(np.int64)
        np.testing.assert_array_equal(r.level, ref)
        assert r.depth == ref.max()


def test_bfs_exhaustive_three_vertices():
    """Every digraph on 3 vertices, self-loops included (2^9), every source,
    against levels from boolean matrix powers."""
    pairs = [(u, v) for u in range(3) for v in range(3)]
    for mask in range(1 << len(pairs)):
        es = [pairs[i] for i in range(len(pairs)) if mask >> i & 1]
        g = graphgen.from_edges(3, [e[0] for e in es], [e[1] for e in es], drop_self=False)
        A = _pins.dense_adjacency(3, g.row_ptr, g.col_idx)
        for s in range(3):
            np.testing.assert_array_equal(oracle.bfs(g.row_ptr, g.col_idx, s).level,
                                          _pins.brute_levels(A, s), err_msg=str((es, s)))


def test_bfs_chain_follows_edge_direction():
    n = 37
    g = graphgen.chain(n)
    np.testing.assert_array_equal(oracle.bfs(g.row_ptr, g.col_idx, 0).level, np.arange(n))
    lv = oracle.bfs(g.row_ptr, g.col_idx, 10).level
    np.testing.assert_array_equal(lv, np.where(np.arange(n) >= 10, np.arange(n) - 10, -1))
    u = np.arange(n - 1)
    rev = graphgen.from_edges(n, u + 1, u)  # i+1 -> i
    lv = oracle.bfs(rev.row_ptr, rev.col_idx, 0).level
    assert lv[0] == 0 and np.all(lv[1:] == -1)
    np.testing.assert_array_equal(oracle.bfs(rev.row_ptr, rev.col_idx, n - 1).level,
                                  n - 1 - np.arange(n))


def test_bfs_cycle_and_stars():
    n = 41
    g = graphgen.cycle(n)
    for s in (0, 17):
        np.testing.assert_array_equal(oracle.bfs(g.row_ptr, g.col_idx, s).level,
                                      (np.arange(n) - s) % n)
    out = graphgen.star(n, inward=False)
    r = oracle.bfs(out.row_ptr, out.col_idx, 0)
    assert r.level[0] == 0 and np.all(r.level[1:] == 1) and r.depth == 1
    assert r.edges_scanned == n - 1
    r = oracle.bfs(out.row_ptr, out.col_idx, 5)
    assert r.level[5] == 0 and np.count_nonzero(r.level >= 0) == 1 and r.depth == 0
    inw = graphgen.star(n, inward=True)
    lv = oracle.bfs(inw.row_ptr, inw.col_idx, 3).level
    expect = np.full(n, -1)
    expect[3], expect[0] = 0, 1
    np.testing.assert_array_equal(lv, expect)


@pytest.mark.parametrize("nx,ny", [(7, 5), (64, 64), (1024, 1024)])
def test_bfs_grid_manhattan(nx, ny):
    g = graphgen.grid2d(nx, ny)
    v = np.arange(nx * ny)
    x, y = v % nx, v // nx
    r = oracle.bfs(g.row_ptr, g.col_idx, 0)
    np.testing.assert_array_equal(r.level, x + y)
    assert r.depth == nx + ny - 2  # 2046 at 1024 x 1024
    assert r.edges_scanned == g.m
    cx, cy = nx // 2, ny // 3
    r = oracle.bfs(g.row_ptr, g.col_idx, cx + nx * cy)
    np.testing.assert_array_equal(r.level, np.abs(x - cx) + np.abs(y - cy))


@pytest.mark.parametrize("g", RANDOM[2:], ids=lambda g: g.name)
def test_bfs_invariants(g):
    """Reached edges never skip a level; every reached vertex but the source
    has an in-neighbour one level up; edges_scanned = out-degrees reached."""
    s = 1
    r = oracle.bfs(g.row_ptr, g.col_idx, s)
    src, dst = g.edges()
    lu, lv = r.level[src], r.level[dst]
    hit = lu >= 0
    assert np.all(lv[hit] >= 0) and np.all(lv[hit] <= lu[hit] + 1)
    parent_ok = np.zeros(g.n, dtype=bool)
    parent_ok[dst[hit & (lv == lu + 1)]] = True
    reached = np.flatnonzero(r.level >= 0)
    assert np.all(parent_ok[reached[reached != s]])
    assert r.edges_scanned == int(g.out_degree()[r.level >= 0].sum())


def test_bfs_rejects_bad_source():
    g = graphgen.tiny()
    for s in (-1, g.n):
        with pytest.raises(ValueError):
            oracle.bfs(g.row_ptr, g.col_idx, s)


def test_bfs_single_and_empty():
    g = graphgen.single()
    r = oracle.bfs(g.row_ptr, g.col_idx, 0)
    assert list(r.level) == [0] and r.depth == 0 and r.edges_scanned == 0
    g = graphgen.empty(6)
    r = oracle.bfs(g.row_ptr, g.col_idx, 4)
    assert list(r.level) == [-1, -1, -1, -1, 0, -1]


# ---------------------------------------------------------------------- WCC

@pytest.mark.parametrize("g", RANDOM, ids=lambda g: g.name)
def test_wcc_matches_scipy_weak_components(g):
    label, k = oracle.wcc(g.row_ptr, g.col_idx)
    nc, comp = csgraph.connected_components(_scipy_matrix(g), directed=True, connection="weak")
    np.testing.assert_array_equal(label, _min_id_labels(comp))
    assert k == nc == np.count_nonzero(label == np.arange(g.n))


def test_wcc_exhaustive_three_vertices():
    pairs = [(u, v) for u in range(3) for v in range(3)]
    for mask in range(1 << len(pairs)):
        es = [pairs[i] for i in range(len(pairs)) if mask >> i & 1]
        g = graphgen.from_edges(3, [e[0] for e in es], [e[1] for e in es], drop_self=False)
        A = _pins.dense_adjacency(3, g.row_ptr, g.col_idx)
        np.testing.assert_array_equal(oracle.wcc(g.row_ptr, g.col_idx)[0],
                                      _pins.brute_weak_labels(A), err_msg=str(es))


def test_wcc_closed_forms():
    g = graphgen.empty(9)
    label, k = oracle.wcc(g.row_ptr, g.col_idx)
    np.testing.assert_array_equal(label, np.arange(9))
    assert k == 9
    for g in (graphgen.cycle(30), graphgen.star(30, True), graphgen.star(30, False),
              graphgen.grid2d(16, 9), graphgen.complete(5), graphgen.single()):
        label, k = oracle.wcc(g.row_ptr, g.col_idx)
        assert k == 1 and np.all(label == 0), g.name
    n = 25
    u = np.arange(n - 1)
    rev = graphgen.from_edges(n, u + 1, u)  # only backward edges: still one component
    assert np.all(oracle.wcc(rev.row_ptr, rev.col_idx)[0] == 0)
    # two disjoint cycles on interleaved ids: evens and odds
    ev, od = np.arange(0, 20, 2), np.arange(1, 20, 2)
    g = graphgen.from_edges(20, np.concatenate([ev, od]),
                            np.concatenate([np.roll(ev, -1), np.roll(od, -1)]))
    label, k = oracle.wcc(g.row_ptr, g.col_idx)
    assert k == 2
    np.testing.assert_array_equal(label, np.arange(20) % 2)


@pytest.mark.parametrize("g", RANDOM, ids=lambda g: g.name)
def test_wcc_ignores_direction(g):
    in_rp, in_ci = oracle.transpose(g.row_ptr, g.col_idx)
    np.testing.assert_array_equal(oracle.wcc(g.row_ptr, g.col_idx)[0],
                                  oracle.wcc(in_rp, in_ci)[0])
