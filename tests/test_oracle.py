"""Pins of the CPU oracle against things other than itself: a library sort,
brute-force enumeration, dense linear solves, closed forms, and the invariants
stated on the pages ("100 Days of GPU", Day 40: the unit sum after every pass
and the total of the variant without dangling redistribution)."""
import itertools
import json
import os

import numpy as np
import pytest

import graphgen
import oracle
from tests import _pins

D = 0.85


# ------------------------------------------------------------------ transpose

def _lexsort_transpose(g):
    src, dst = g.edges()
    order = np.lexsort((src, dst))  # by v, then by u
    in_ci = src[order]
    in_rp = np.zeros(g.n + 1, dtype=np.int64)
    np.add.at(in_rp, dst + 1, 1)
    return np.cumsum(in_rp), in_ci


@pytest.mark.parametrize("g", [graphgen.tiny(), graphgen.single(), graphgen.empty(5),
                               graphgen.random_graph(1000, 7000, 3),
                               graphgen.random_graph(300, 9000, 4, dedup=False, drop_self=False),
                               graphgen.rmat(12), graphgen.citation()],
                         ids=lambda g: g.name)
def test_transpose_matches_lexicographic_sort(g):
    in_rp, in_ci = oracle.transpose(g.row_ptr, g.col_idx)
    ref_rp, ref_ci = _lexsort_transpose(g)
    np.testing.assert_array_equal(in_rp, ref_rp)
    np.testing.assert_array_equal(in_ci, ref_ci)
    assert in_rp[-1] == g.m
    np.testing.assert_array_equal(np.diff(in_rp), np.bincount(g.col_idx, minlength=g.n))


def test_transpose_exhaustive_four_vertices():
    """Every digraph on 4 vertices without self-loops (2^12 of them)."""
    pairs = [(u, v) for u in range(4) for v in range(4) if u != v]
    for mask in range(1 << len(pairs)):
        es = [pairs[i] for i in range(len(pairs)) if mask >> i & 1]
        g = graphgen.from_edges(4, [e[0] for e in es], [e[1] for e in es])
        in_rp, in_ci = oracle.transpose(g.row_ptr, g.col_idx)
        b_rp, b_ci = _pins.brute_transpose(4, g.row_ptr, g.col_idx)
        assert np.array_equal(in_rp, b_rp) and np.array_equal(in_ci, b_ci), es


def test_transpose_exhaustive_three_vertices_with_loops_and_multi_edges():
    pairs = [(u, v) for u in range(3) for v in range(3)]
    for mask in range(1 << len(pairs)):
        es = [pairs[i] for i in range(len(pairs)) if mask >> i & 1]
        es = es + es[: len(es) // 2]  # some parallel edges
        g = graphgen.from_edges(3, [e[0] for e in es], [e[1] for e in es], dedup=False,
                                drop_self=False)
        in_rp, in_ci = oracle.transpose(g.row_ptr, g.col_idx)
        b_rp, b_ci = _pins.brute_transpose(3, g.row_ptr, g.col_idx)
        assert np.array_equal(in_rp, b_rp) and np.array_equal(in_ci, b_ci), es


def test_transpose_twice_is_identity():
    g = graphgen.rmat(11)
    in_rp, in_ci = oracle.transpose(g.row_ptr, g.col_idx)
    rp2, ci2 = oracle.transpose(in_rp, in_ci)
    np.testing.assert_array_equal(rp2, g.row_ptr)
    np.testing.assert_array_equal(ci2, g.col_idx)


def test_transpose_of_symmetric_stencil_is_itself():
    g = graphgen.stencil27(7, 5, 6)
    in_rp, in_ci = oracle.transpose(g.row_ptr, g.col_idx)
    np.testing.assert_array_equal(in_rp, g.row_ptr)
    np.testing.assert_array_equal(in_ci, g.col_idx)


def test_transpose_rejects_malformed_csr():
    rp = np.array([0, 2, 1, 3], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.transpose(rp, np.array([0, 1, 2], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.transpose(np.array([0, 1], dtype=np.int32), np.array([5], dtype=np.int32))


# --------------------------------------------------- fixed point: dense solves

def _converged(g, d=D):
    return oracle.pagerank(g.row_ptr, g.col_idx, d=d, tol=0.0, max_iter=400).x


def test_dense_solve_exhaustive_three_vertices_with_self_loops():
    """All 512 digraphs on 3 vertices, self-loops allowed."""
    pairs = [(u, v) for u in range(3) for v in range(3)]
    for mask in range(1 << len(pairs)):
        es = [pairs[i] for i in range(len(pairs)) if mask >> i & 1]
        g = graphgen.from_edges(3, [e[0] for e in es], [e[1] for e in es], drop_self=False)
        x = _converged(g)
        ref = _pins.dense_pagerank(3, g.row_ptr, g.col_idx)
        assert np.abs(x - ref).max() <= 1e-12, es


@pytest.mark.parametrize("seed", range(40))
def test_dense_solve_random_small_graphs(seed):
    n = 2 + seed % 9  # 2 .. 10 vertices
    g = graphgen.random_graph(n, 3 * n, seed, dedup=bool(seed % 2), drop_self=bool(seed % 3))
    for d in (0.85, 0.5, 0.99):
        x = oracle.pagerank(g.row_ptr, g.col_idx, d=d, max_iter=3000 if d > 0.9 else 400).x
        ref = _pins.dense_pagerank(n, g.row_ptr, g.col_idx, d)
        assert np.abs(x - ref).max() <= 1e-12


def test_dense_solve_antv_simple_dataset(golden_dir):
    data = json.load(open(os.path.join(golden_dir, "antv_simple_dataset.json")))
    ids = {name: i for i, name in enumerate(data["nodes"])}
    src = [ids[a] for a, _ in data["edges"]]
    dst = [ids[b] for _, b in data["edges"]]
    g = graphgen.from_edges(len(ids), src, dst)
    assert g.m == 17 and g.n_dangling() == 1 and g.out_degree()[ids["A"]] == 0
    x = _converged(g)
    ref = _pins.dense_pagerank(g.n, g.row_ptr, g.col_idx)
    assert np.abs(x - ref).max() <= 1e-12
    assert oracle.top_k(x, 1)[0] == ids["B"]  # B receives the most rank


# ---------------------------------------------------------------- closed forms

def test_cycle_is_uniform_every_iteration():
    g = graphgen.cycle(97)
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=30)
    assert np.abs(r.x - 1 / 97).max() <= 1e-15
    assert r.l1_trace.max() <= 1e-13


@pytest.mark.parametrize("g", [graphgen.empty(13), graphgen.complete(9)], ids=lambda g: g.name)
def test_no_edges_and_complete_digraph_are_uniform(g):
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=20)
    assert np.abs(r.x - 1 / g.n).max() <= 1e-15


def test_single_vertex_keeps_all_rank():
    g = graphgen.single()
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=5)
    assert r.x.tolist() == [1.0]


@pytest.mark.parametrize("N", [2, 3, 10001])
def test_star_closed_forms(N):
    gi = graphgen.star(N, inward=True)
    h, l = _pins.star_in_closed_form(N, D)
    x = _converged(gi)
    # the hub sums N-1 terms in double: allow N ulps relative
    assert abs(x[0] - h) <= N * 2.3e-16 * h and np.abs(x[1:] - l).max() <= 1e-15
    go = graphgen.star(N, inward=False)
    h, l = _pins.star_out_closed_form(N, D)
    x = _converged(go)
    assert abs(x[0] - h) <= N * 2.3e-16 * h and np.abs(x[1:] - l).max() <= 1e-15


@pytest.mark.parametrize("n", [2, 5, 8192])
def test_chain_closed_form(n):
    g = graphgen.chain(n)
    x = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=max(400, n + 300)).x
    np.testing.assert_allclose(x, _pins.chain_closed_form(n, D), rtol=1e-11, atol=1e-17)


# ------------------------------------------------------------------ invariants

SMALL = [graphgen.tiny(), graphgen.nodangling(), graphgen.dangling(), graphgen.star(10001),
         graphgen.chain(8192), graphgen.rmat(10), graphgen.citation()]


@pytest.mark.parametrize("g", SMALL, ids=lambda g: g.name)
def test_unit_sum_after_every_pass(g):
    """Day 40: the ranks sum to 1 after every pass."""
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=100)
    assert np.abs(r.sum_trace - 1).max() <= 1e-12


@pytest.mark.parametrize("g", SMALL, ids=lambda g: g.name)
def test_l1_trace_contracts(g):
    """x_{t+1} - x_t = d M (x_t - x_{t-1}) with M column-stochastic."""
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=60)
    l1 = r.l1_trace
    assert np.all(l1[1:] <= D * l1[:-1] + 1e-15)


@pytest.mark.parametrize("g", [graphgen.tiny(), graphgen.dangling(), graphgen.star(101),
                               graphgen.citation()], ids=lambda g: g.name)
def test_dropped_dangling_total_and_fixed_point(g, golden_dir):
    """Day 40 exercise: without redistribution S' = (1-d) + d (S - D); the
    fixed-point total is 1 - D d/(1-d) (multiplier 17/3 at d = 0.85) and the
    broken vector is the correct one times that total."""
    ex = json.load(open(os.path.join(golden_dir, "day40_exercise.json")))
    d = ex["damping"]
    mult = ex["fixed_point_multiplier"]["num"] / ex["fixed_point_multiplier"]["den"]
    assert abs(d / (1 - d) - mult) <= 1e-12
    r = oracle.pagerank(g.row_ptr, g.col_idx, d=d, max_iter=400, drop_dangling=True)
    # the mass the dropped term would have carried, from the same input vectors
    xs = [np.full(g.n, 1.0 / g.n)]
    S_prev = 1.0
    for t in range(5):
        rt = oracle.pagerank(g.row_ptr, g.col_idx, d=d, max_iter=t + 1, drop_dangling=True)
        dang = g.out_degree() == 0
        Dm = xs[-1][dang].sum()
        assert abs(rt.sum_trace[-1] - ((1 - d) + d * (S_prev - Dm))) <= 1e-13
        if t == 0:
            assert abs(rt.sum_trace[-1] - (1 - d * Dm)) <= 1e-13
        S_prev = rt.sum_trace[-1]
        xs.append(rt.x)
    S = r.x.sum()
    Dstar = r.x[g.out_degree() == 0].sum()
    assert abs(S - (1 - Dstar * mult)) <= 1e-12
    assert S < 1.0
    good = oracle.pagerank(g.row_ptr, g.col_idx, d=d, max_iter=400).x
    np.testing.assert_allclose(r.x, S * good, rtol=1e-10, atol=1e-17)
    # order unchanged (compare ranks where the correct values are not tied)
    assert np.array_equal(np.argsort(-good, kind="stable"), np.argsort(-r.x, kind="stable")) or \
        np.allclose(np.sort(good), np.sort(r.x / S), rtol=1e-10)


def test_nodangling_graph_unaffected_by_dropping():
    g = graphgen.nodangling()
    a = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=50)
    b = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=50, drop_dangling=True)
    np.testing.assert_array_equal(a.x, b.x)


def test_dangling_mass_is_taken_from_the_input_vector():
    """Iteration 1 starts from 1/n, so D_1 = (#dangling)/n exactly."""
    g = graphgen.dangling()
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=3)
    assert abs(r.dmass_trace[0] - 400 / 4096) <= 1e-15
    r1 = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=1)
    assert abs(r.dmass_trace[1] - r1.x[g.out_degree() == 0].sum()) <= 1e-15


def test_one_iteration_by_hand_on_tiny():
    """x1 from the uniform start, worked by hand on the 6-vertex graph
    0->{1,2} 1->{2,3} 2->{0} 3->{4,5} 4->{0,5} 5->{} (5 dangling)."""
    g = graphgen.tiny()
    n, d = 6, D
    c = 1.0 / n
    base = (1 - d) / n + d * (c / n)  # D = x[5] = 1/6
    hand = np.array([
        base + d * (c / 1 + c / 2),  # 0 <- 2 (deg 1), 4 (deg 2)
        base + d * (c / 2),          # 1 <- 0
        base + d * (c / 2 + c / 2),  # 2 <- 0, 1
        base + d * (c / 2),          # 3 <- 1
        base + d * (c / 2),          # 4 <- 3
        base + d * (c / 2 + c / 2),  # 5 <- 3, 4
    ])
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=1)
    np.testing.assert_allclose(r.x, hand, rtol=0, atol=1e-16)
    assert abs(r.l1_trace[0] - np.abs(hand - c).sum()) <= 1e-15


# ---------------------------------------------------------------- stop rule

def test_stop_rule_counts_the_iteration_that_meets_tol():
    g = graphgen.citation()
    full = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=100)
    tol = 1e-6
    first = int(np.argmax(full.l1_trace < tol)) + 1
    r = oracle.pagerank(g.row_ptr, g.col_idx, tol=tol, max_iter=100)
    assert r.iterations == first
    assert r.l1_trace[-1] < tol and np.all(r.l1_trace[:-1] >= tol)
    np.testing.assert_array_equal(r.l1_trace, full.l1_trace[:first])
    capped = oracle.pagerank(g.row_ptr, g.col_idx, tol=tol, max_iter=first - 1)
    assert capped.iterations == first - 1


def test_warm_start_from_fixed_point_stays_put():
    g = graphgen.rmat(9)
    x = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=300).x
    r = oracle.pagerank(g.row_ptr, g.col_idx, max_iter=2, x0=x)
    assert r.l1_trace.max() <= 1e-14


def test_ranking_breaks_ties_by_id():
    x = np.array([0.1, 0.3, 0.3, 0.2, 0.1])
    assert oracle.ranking(x).tolist() == [1, 2, 3, 0, 4]


def test_rejects_bad_arguments():
    g = graphgen.tiny()
    with pytest.raises(ValueError):
        oracle.pagerank(g.row_ptr, g.col_idx, d=1.5)
    with pytest.raises(ValueError):
        oracle.pagerank(g.row_ptr, g.col_idx, max_iter=0)


# ------------------------------------------------------------ sparse product
# "A Pedagogical Introduction to Porting a Conjugate Gradient Solver to CUDA":
# y[i] = sum over the stored entries j of row i of vals[j] * x[cols[j]].

U = 2.0 ** -53  # unit roundoff of binary64


def _dense(A):
    M = np.zeros((A.n_rows, A.n_cols), dtype=np.float64)
    rows = np.repeat(np.arange(A.n_rows), A.row_lengths())
    np.add.at(M, (rows, A.col_idx), A.vals)
    return M


@pytest.mark.parametrize("shape", [(300, 300), (257, 90), (60, 513)], ids=str)
def test_spmv_integer_entries_match_dense_product_exactly(shape):
    # Small integers: every product and partial sum is an integer far below
    # 2^53, so the floating-point result is exact and must equal the int64
    # dense product.  A rectangular shape makes A^T x impossible to confuse
    # with A x.
    n_rows, n_cols = shape
    lengths = graphgen.splitmix_u64(5, np.arange(n_rows, dtype=np.uint64)) % np.uint64(41)
    A = graphgen.matrix_from_lengths(lengths, n_cols, seed=9, int_values=True)
    x = graphgen.small_ints(n_cols, 77)
    dense = _dense(A).astype(np.int64) @ x.astype(np.int64)
    y = oracle.spmv(A.row_ptr, A.col_idx, A.vals, x)
    np.testing.assert_array_equal(y, dense.astype(np.float64))
    assert np.count_nonzero(y) > n_rows // 2


def test_spmv_exact_sum_within_rounding_bound():
    # Each row's exact rational value sum_j a_j x_j; a k-term sum of rounded
    # products differs from it by at most gamma_k * sum_j |a_j x_j| with
    # gamma_k = k u / (1 - k u) (standard forward error bound).
    from fractions import Fraction
    lengths = [0, 1, 2, 3, 7, 31, 64, 65, 200]
    A = graphgen.matrix_from_lengths(lengths, 500, seed=21)
    x = graphgen.uniform(500, 22) * 1e3
    y = oracle.spmv(A.row_ptr, A.col_idx, A.vals, x)
    for i, k in enumerate(lengths):
        s, e = A.row_ptr[i], A.row_ptr[i + 1]
        terms = [Fraction(float(a)) * Fraction(float(x[c])) for a, c in zip(A.vals[s:e], A.col_idx[s:e])]
        exact = sum(terms, Fraction(0))
        mag = float(sum(abs(t) for t in terms))
        gamma = k * U / (1 - k * U)
        assert abs(Fraction(float(y[i])) - exact) <= Fraction(gamma * mag) + Fraction(0), (i, k)


def test_spmv_identity_and_diagonal():
    n = 1000
    x = graphgen.uniform(n, 3)
    eye = graphgen.Matrix("eye", np.arange(n + 1), np.arange(n), np.ones(n), n)
    np.testing.assert_array_equal(oracle.spmv(eye.row_ptr, eye.col_idx, eye.vals, x), x)
    d = graphgen.uniform(n, 4)
    diag = graphgen.Matrix("diag", np.arange(n + 1), np.arange(n), d, n)
    np.testing.assert_array_equal(oracle.spmv(diag.row_ptr, diag.col_idx, diag.vals, x), d * x)
    # a permutation matrix gathers: y[i] = x[p[i]]
    p = np.argsort(graphgen.splitmix_u64(8, np.arange(n, dtype=np.uint64)))
    perm = graphgen.Matrix("perm", np.arange(n + 1), p, np.ones(n), n)
    np.testing.assert_array_equal(oracle.spmv(perm.row_ptr, perm.col_idx, perm.vals, x), x[p])


def test_spmv_empty_rows_and_empty_matrices():
    A = graphgen.matrix_from_lengths([0, 3, 0, 0, 2, 0], 4, seed=1)
    x = graphgen.uniform(4, 2)
    y = oracle.spmv(A.row_ptr, A.col_idx, A.vals, x)
    assert y[0] == 0.0 and y[2] == 0.0 and y[3] == 0.0 and y[5] == 0.0
    assert not np.signbit(y[[0, 2, 3, 5]]).any()  # a sum that starts from +0.0
    assert oracle.spmv(np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0), x).size == 0
    z = oracle.spmv(np.zeros(6, np.int32), np.zeros(0, np.int32), np.zeros(0), x)
    np.testing.assert_array_equal(z, np.zeros(5))


@pytest.mark.parametrize("dims", [(5, 5, 5), (7, 4, 3), (1, 1, 9), (1, 1, 1)], ids=str)
def test_spmv_stencil_operator_on_ones_closed_form(dims):
    # -1 per neighbour and 27 on the diagonal: (A 1)[p] = 27 - k(p), where
    # k(p) counts the in-grid points at Chebyshev distance 1, the product of
    # (number of in-grid offsets -1, 0, +1) per axis minus the point itself.
    nx, ny, nz = dims
    A = graphgen.stencil_matrix(nx, ny, nz)
    y = oracle.spmv(A.row_ptr, A.col_idx, A.vals, np.ones(A.n_cols))
    zz, yy, xx = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")

    def offsets(c, size):  # in-grid offsets among -1, 0, +1 along one axis
        return 1 + (c > 0) + (c < size - 1)

    k = offsets(xx, nx) * offsets(yy, ny) * offsets(zz, nz) - 1
    np.testing.assert_array_equal(y, (27.0 - k).ravel())
    if min(dims) >= 3:
        assert (y == 1.0).sum() == (nx - 2) * (ny - 2) * (nz - 2)


def test_spmv_linearity():
    A = graphgen.matrix_of_graph(graphgen.rmat(10), seed=5)
    x, z = graphgen.uniform(A.n_cols, 6), graphgen.uniform(A.n_cols, 7)
    lhs = oracle.spmv(A.row_ptr, A.col_idx, A.vals, 2.0 * x - 0.5 * z)
    rhs = 2.0 * oracle.spmv(A.row_ptr, A.col_idx, A.vals, x) - 0.5 * oracle.spmv(
        A.row_ptr, A.col_idx, A.vals, z)
    scale = oracle.spmv(A.row_ptr, A.col_idx, np.abs(A.vals), 2.0 * np.abs(x) + 0.5 * np.abs(z))
    k = A.row_lengths().max() + 2
    assert np.all(np.abs(lhs - rhs) <= 3 * k * U * scale + 1e-300)


def test_spmv_rejects_malformed_csr():
    x = np.ones(3)
    with pytest.raises(ValueError):
        oracle.spmv(np.array([0, 2, 1]), np.array([0, 1]), np.ones(2), x)   # decreasing
    with pytest.raises(ValueError):
        oracle.spmv(np.array([0, 1, 2]), np.array([0, 3]), np.ones(2), x)   # column >= n_cols
    with pytest.raises(ValueError):
        oracle.spmv(np.array([1, 2]), np.array([0, 1]), np.ones(2), x)      # row_ptr[0] != 0
    with pytest.raises(ValueError):
        oracle.spmv(np.array([0, 2]), np.array([0, 1]), np.ones(3), x)      # vals length
