"""The seeded input generators: shapes of the pages' workloads, determinism,
and CSR well-formedness (rows sorted, no duplicates, no self-loops)."""
import json
import os

import numpy as np
import pytest

import graphgen


def _well_formed(g, allow_self=False):
    rp, ci = g.row_ptr.astype(np.int64), g.col_idx.astype(np.int64)
    assert rp[0] == 0 and rp[-1] == g.m and np.all(np.diff(rp) >= 0)
    assert g.m == 0 or (ci.min() >= 0 and ci.max() < g.n)
    src = np.repeat(np.arange(g.n), np.diff(rp))
    same_row = src[1:] == src[:-1]
    assert np.all(ci[1:][same_row] > ci[:-1][same_row]), "rows not strictly ascending"
    if not allow_self:
        assert not np.any(src == ci)


def test_day40_case_sizes(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "day40_correctness_cases.json")))["cases"]
    built = {"tiny": graphgen.tiny(), "single": graphgen.single(),
             "nodangling": graphgen.nodangling(), "dangling": graphgen.dangling(),
             "star": graphgen.star(10001), "chain": graphgen.chain(8192)}
    for c in cases:
        g = built[c["name"]]
        assert (g.n, g.m) == (c["n"], c["nnz"]), c["name"]
        _well_formed(g)
    assert built["tiny"].n_dangling() >= 1
    assert built["nodangling"].n_dangling() == 0
    assert built["dangling"].n_dangling() == 400


def test_citation_like_shape(golden_dir):
    real = json.load(open(os.path.join(golden_dir, "day40_correctness_cases.json")))["real_graph"]
    g = graphgen.citation()
    _well_formed(g)
    assert g.n == real["n"] and g.n_dangling() == real["dangling"]
    mean = g.m / (g.n - g.n_dangling())
    assert 11.0 < mean < 13.0  # geometric with mean 12
    assert abs(g.m - real["nnz"]) / real["nnz"] < 0.05
    indeg = np.bincount(g.col_idx, minlength=g.n)
    assert indeg.max() > 5 * indeg.mean()  # preferential attachment skews in-degree


def test_stencil_counts():
    g = graphgen.stencil27(100)
    assert g.n == 1_000_000 and g.m == 298 ** 3 - 100 ** 3 == 25_463_592
    assert g.n_dangling() == 0
    deg = g.out_degree()
    assert deg.min() == 7 and deg.max() == 26
    small = graphgen.stencil27(4, 3, 5)
    _well_formed(small)
    assert small.m == (3 * 4 - 2) * (3 * 3 - 2) * (3 * 5 - 2) - 60


def test_stencil_matrix_layout():
    A = graphgen.stencil_matrix(6, 5, 4)
    assert A.n_rows == A.n_cols == 120
    assert A.nnz == (3 * 6 - 2) * (3 * 5 - 2) * (3 * 4 - 2)
    rows = np.repeat(np.arange(A.n_rows), A.row_lengths())
    assert np.all(np.diff(A.col_idx.astype(np.int64))[np.diff(rows) == 0] > 0)  # ascending
    diag = A.col_idx == rows
    assert np.array_equal(np.bincount(rows[diag], minlength=A.n_rows), np.ones(A.n_rows))
    assert np.all(A.vals[diag] == 27.0) and np.all(A.vals[~diag] == -1.0)
    g = graphgen.stencil27(6, 5, 4)
    assert np.array_equal(A.col_idx[~diag], g.col_idx)  # the graph's edges, in order
    R = graphgen.stencil_matrix(6, 5, 4, values="random", seed=3)
    assert np.array_equal(R.col_idx, A.col_idx) and np.all(np.abs(R.vals) < 1.0)


def test_rmat_deterministic_and_well_formed():
    a, b = graphgen.rmat(14), graphgen.rmat(14)
    np.testing.assert_array_equal(a.row_ptr, b.row_ptr)
    np.testing.assert_array_equal(a.col_idx, b.col_idx)
    _well_formed(a)
    c = graphgen.rmat(14, seed=99)
    assert not np.array_equal(a.col_idx[:1000], c.col_idx[:1000])
    # skew: vertex 0 (all-zero bits) is the largest hub in both directions
    indeg = np.bincount(a.col_idx, minlength=a.n)
    assert indeg.argmax() == 0 and a.out_degree().argmax() == 0
    assert indeg.max() > 100 * indeg.mean()
    assert a.m < 32 << 14


def test_rmat_quadrant_frequencies():
    """Top bit of (u, v) follows (a, b, c, d) = (.57, .19, .19, .05) before cleanup."""
    g = graphgen.rmat(10, edge_factor=64)
    src, dst = g.edges()
    top_u, top_v = src >> 9, dst >> 9
    frac = np.array([np.mean((top_u == i) & (top_v == j)) for i in (0, 1) for j in (0, 1)])
    # dedup removes more edges from the dense (0,0) quadrant, so allow slack
    assert frac.argmax() == 0 and frac.argmin() == 3
    assert abs(frac[1] - frac[2]) < 0.02


def test_splitmix_python_matches_c():
    lib = graphgen._lib()
    k = np.arange(50, dtype=np.uint64)
    py = graphgen.splitmix_u64(12345, k)
    c = np.array([lib.gg_draw_u64(12345, int(i)) for i in k], dtype=np.uint64)
    np.testing.assert_array_equal(py, c)


def test_from_edges_dedup_and_order():
    g = graphgen.from_edges(4, [3, 0, 0, 3, 2, 2], [1, 2, 1, 1, 2, 0])
    assert g.row_ptr.tolist() == [0, 2, 2, 3, 4]
    assert g.col_idx.tolist() == [1, 2, 0, 1]
    with pytest.raises(ValueError):
        graphgen.from_edges(2, [0], [2])


def test_relabel_is_the_same_graph_under_the_permutation():
    g = graphgen.rmat(11)
    r = graphgen.relabel(g, 31)
    perm = graphgen.relabel_permutation(g.n, 31)
    assert sorted(perm.tolist()) == list(range(g.n))
    src, dst = g.edges()
    s2, d2 = r.edges()
    assert r.m == g.m
    assert set(zip(perm[src].tolist(), perm[dst].tolist())) == set(zip(s2.tolist(), d2.tolist()))
    # rows sorted, no duplicates
    for u in range(r.n):
        row = r.col_idx[r.row_ptr[u]:r.row_ptr[u + 1]]
        assert np.all(np.diff(row) > 0)


def test_edge_batch_applies_deletions_and_insertions():
    g = graphgen.rmat(10)
    dele, u, v = graphgen.edge_batch(g, 300, 500, seed=4)
    assert dele.size == 300 and np.all(np.diff(dele) > 0) and dele.max() < g.m
    assert u.size == 500 and u.max() < g.n and v.max() < g.n
    h = graphgen.apply_batch(g, dele, u, v)
    src, dst = g.edges()
    keep = np.ones(g.m, bool)
    keep[dele] = False
    want = set(zip(src[keep].tolist(), dst[keep].tolist()))
    want |= {(a, b) for a, b in zip(u.tolist(), v.tolist()) if a != b}
    s2, d2 = h.edges()
    assert set(zip(s2.tolist(), d2.tolist())) == want and h.m == len(want)
    # deterministic
    d_again, u_again, v_again = graphgen.edge_batch(g, 300, 500, seed=4)
    assert np.array_equal(dele, d_again) and np.array_equal(u, u_again)
    # a batch with nothing in it leaves the graph as it was
    same = graphgen.apply_batch(g, np.zeros(0, np.int64), np.zeros(0, np.int32),
                                np.zeros(0, np.int32))
    assert np.array_equal(same.row_ptr, g.row_ptr) and np.array_equal(same.col_idx, g.col_idx)
