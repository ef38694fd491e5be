"""GPU parity of breadth-first search (pr_bfs) and weakly connected
components (pr_wcc) against the CPU oracle on the same seeded graphs.

Both results are integers and unique ("gpu-graph-study", sections "Traversal
(BFS / WCC)" and "Traversal T4 -- degree-bucketed BFS / WCC": the level of a
vertex is its shortest-path distance from the source, and the label of a
vertex is the smallest id of its weak component), so the bar is bit-exact:
every level, the depth, the out-edges scanned, every label and the number of
components.  Which edge claimed a vertex, which direction a level took, and
the shape of the trees linked on the way, are not outputs and are not
compared.  Every case runs twice: with the out-edge CSR alone (top-down
levels; every out-edge linked), and with the in-edge CSR from pr_transpose
as well (bottom-up levels where the frontier is large; the giant tree's
vertices skipped)."""
import numpy as np
import pytest

import graphgen
import oracle
from tests import _cases

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def prx():
    import pagerank_power_iteration_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()  # fail loudly if the HIP library is missing
    return m


def _hub_graph():
    """Rows on both sides of the 256-edge hub threshold and of the 2048-edge
    chunk size, a 70,000-edge hub, and a tail of short rows."""
    n = 80_000
    lens = [0, 1, 63, 64, 65, 255, 256, 257, 2047, 2048, 2049, 4097, 70_000, 3, 0, 17]
    src, dst = [], []
    for u, L in enumerate(lens):
        t = (np.arange(L, dtype=np.int64) * 7919 + u * 104_729 + 1) % n
        t = np.unique(t[t != u])
        src.append(np.full(t.size, u))
        dst.append(t)
    rest = np.arange(len(lens), n, dtype=np.int64)
    src.append(rest)
    dst.append((rest * 31 + 5) % n)
    return graphgen.from_edges(n, np.concatenate(src), np.concatenate(dst), name="hubs")


def _bottom_up_graph():
    """Source 0 reaches 3000 vertices that together have 60,000 out-edges, so
    the search turns bottom-up at level 1; ten unvisited vertices have 3000
    in-edges each (hub in-rows), five of them with a level-1 parent (vertex
    1, the first entry of their in-rows) and five with none."""
    n = 100_000
    rng = graphgen.splitmix_u64(77, np.arange(200_000, dtype=np.uint64))
    src = [np.zeros(3000, dtype=np.int64)]
    dst = [np.arange(1, 3001)]
    lvl1 = np.repeat(np.arange(1, 3001), 20)
    src.append(lvl1)
    dst.append(3001 + (rng[:lvl1.size] % np.uint64(n - 3001)).astype(np.int64))
    for h in range(10):
        srcs = 3001 + (rng[60_000 + 3000 * h:63_000 + 3000 * h] % np.uint64(40_000)).astype(np.int64)
        src.append(srcs)
        dst.append(np.full(srcs.size, 50_000 + h))
    src.append(np.ones(5, dtype=np.int64))
    dst.append(50_000 + np.arange(5))
    return graphgen.from_edges(n, np.concatenate(src), np.concatenate(dst), name="bottomup")


def _reversed_chain(n):
    u = np.arange(n - 1)
    return graphgen.from_edges(n, u + 1, u, name=f"rchain{n}")


CASES = [
    graphgen.tiny(), graphgen.single(), graphgen.empty(5), graphgen.chain(3000),
    _reversed_chain(3000), graphgen.cycle(1000), graphgen.star(10_001, inward=True),
    graphgen.star(10_001, inward=False), graphgen.complete(70), graphgen.nodangling(),
    graphgen.dangling(), graphgen.grid2d(64, 48),
    graphgen.random_graph(4097, 40_961, 13, dedup=False, drop_self=False, name="multigraph4097"),
    graphgen.random_graph(70_001, 90_007, 15, name="sparse70001"),
    graphgen.random_graph(70_001, 300_007, 14, name="random70001"),
    graphgen.stencil27(13, 11, 9), graphgen.citation(), graphgen.rmat(14),
    graphgen.rmat(16, edge_factor=16), _hub_graph(), _bottom_up_graph(),
]
MODES = ["out", "out+in"]


def _sources(g):
    out = {0, g.n - 1, g.n // 3}
    deg = g.out_degree()
    if g.m:
        out.add(int(np.argmax(deg)))
    return sorted(out)


def _in_csr(prx, dg, mode):
    return prx.transpose(dg) if mode == "out+in" else None


def _check_bfs(prx, g, dg, s, ws=None, in_csr=None):
    level, depth, scanned = prx.bfs(dg, s, in_csr=in_csr, ws=ws)
    ref = oracle.bfs(g.row_ptr, g.col_idx, s)
    got = _cases.to_np(level)
    if not np.array_equal(got, ref.level):
        bad = np.flatnonzero(got != ref.level)
        raise AssertionError(f"{g.name} source {s}: {bad.size} levels differ, first at "
                             f"{bad[:5].tolist()}: gpu {got[bad[:5]].tolist()} oracle "
                             f"{ref.level[bad[:5]].tolist()}")
    assert depth == ref.depth, (g.name, s, depth, ref.depth)
    assert scanned == ref.edges_scanned, (g.name, s, scanned, ref.edges_scanned)


def _check_wcc(prx, g, dg, ws=None, in_csr=None):
    label, comps = prx.wcc(dg, in_csr=in_csr, ws=ws)
    ref, ref_comps = oracle.wcc(g.row_ptr, g.col_idx)
    got = _cases.to_np(label)
    if not np.array_equal(got, ref):
        bad = np.flatnonzero(got != ref)
        raise AssertionError(f"{g.name}: {bad.size} labels differ, first at {bad[:5].tolist()}: "
                             f"gpu {got[bad[:5]].tolist()} oracle {ref[bad[:5]].tolist()}")
    assert comps == ref_comps


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("g", CASES, ids=lambda g: g.name)
def test_bfs_levels_bit_exact(prx, g, mode):
    print(f"[bfs {mode}] {g.name} n={g.n} m={g.m}", flush=True)
    dg = _cases.gpu_graph(g)
    in_csr = _in_csr(prx, dg, mode)
    for s in _sources(g):
        _check_bfs(prx, g, dg, s, in_csr=in_csr)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("g", CASES, ids=lambda g: g.name)
def test_wcc_labels_bit_exact(prx, g, mode):
    print(f"[wcc {mode}] {g.name} n={g.n} m={g.m}", flush=True)
    dg = _cases.gpu_graph(g)
    _check_wcc(prx, g, dg, in_csr=_in_csr(prx, dg, mode))


@pytest.mark.parametrize("mode", MODES)
def test_bfs_grid_is_2046_levels_deep(prx, mode):
    """The graph study's high-diameter grid: 1024 x 1024, BFS from a corner
    reaches the far corner at level 2046 (closed form: level = x + y)."""
    g = graphgen.grid2d(1024)
    dg = _cases.gpu_graph(g)
    in_csr = _in_csr(prx, dg, mode)
    level, depth, scanned = prx.bfs(dg, 0, in_csr=in_csr)
    v = np.arange(g.n)
    np.testing.assert_array_equal(_cases.to_np(level), v % 1024 + v // 1024)
    assert depth == 2046 and scanned == g.m
    label, comps = prx.wcc(dg, in_csr=in_csr)
    assert comps == 1 and not _cases.to_np(label).any()


@pytest.mark.parametrize("nx, ny, sx, sy", [
    # frontiers of up to 1,536 vertices (more than one per lane of the
    # single-workgroup levels): the centre-left source of the 1024 x 1024 grid
    (1024, 1024, 256, 512),
    # more vertices than the visited bitmap in LDS covers (2^20): those
    # levels claim by compare-and-swap on the level array
    (1100, 1000, 0, 0),
    (1100, 1000, 550, 500),
])
def test_bfs_grid_levels_are_manhattan_distances(prx, nx, ny, sx, sy):
    """On a 4-neighbour grid the BFS level of (x, y) is |x - sx| + |y - sy|
    (closed form), the depth is the largest such distance and every one of
    the grid's out-edges is scanned once."""
    g = graphgen.grid2d(nx, ny)
    print(f"[bfs grid] {g.name} source ({sx}, {sy})", flush=True)
    dg = _cases.gpu_graph(g)
    level, depth, scanned = prx.bfs(dg, sx + nx * sy)
    v = np.arange(g.n)
    want = np.abs(v % nx - sx) + np.abs(v // nx - sy)
    np.testing.assert_array_equal(_cases.to_np(level), want)
    assert depth == want.max() and scanned == g.m


def test_reused_workspace_and_repeats(prx):
    """Calls reuse one workspace; a second search from another source and a
    rerun give the oracle's results again (no state leaks between calls)."""
    g = graphgen.rmat(14)
    dg = _cases.gpu_graph(g)
    in_csr = prx.transpose(dg)
    ws = torch.empty(prx.pr_bfs_workspace_bytes(g.n, g.m), dtype=torch.uint8, device="cuda")
    for s, ic in ((0, None), (5, in_csr), (0, in_csr), (5, None)):
        _check_bfs(prx, g, dg, s, ws, ic)
    ws = torch.empty(prx.pr_wcc_workspace_bytes(g.n, g.m), dtype=torch.uint8, device="cuda")
    for ic in (None, in_csr, in_csr, None):
        _check_wcc(prx, g, dg, ws, ic)


def test_validate_rejects_malformed(prx):
    g = graphgen.tiny()
    bad_col = g.col_idx.copy()
    bad_col[3] = g.n
    bad_rp = g.row_ptr.copy()
    bad_rp[2], bad_rp[3] = bad_rp[3], bad_rp[2]
    good = _cases.gpu_graph(g)
    good_in = prx.transpose(good)
    for rp, ci in ((g.row_ptr, bad_col), (bad_rp, g.col_idx)):
        dg = prx.DeviceGraph.from_csr(rp, ci)
        for graph, in_csr in ((dg, None), (good, (dg.row_ptr, dg.col_idx))):
            with pytest.raises(prx.PrError) as e:
                prx.bfs(graph, 0, in_csr=in_csr, flags=prx.PR_VALIDATE)
            assert e.value.status == prx.PR_ERR_GRAPH
            with pytest.raises(prx.PrError) as e:
                prx.wcc(graph, in_csr=in_csr, flags=prx.PR_VALIDATE)
            assert e.value.status == prx.PR_ERR_GRAPH
    level, depth, _ = prx.bfs(good, 0, in_csr=good_in, flags=prx.PR_VALIDATE)
    np.testing.assert_array_equal(_cases.to_np(level), oracle.bfs(g.row_ptr, g.col_idx, 0).level)


def test_bad_arguments(prx):
    g = graphgen.tiny()
    dg = _cases.gpu_graph(g)
    for s in (-1, g.n):
        with pytest.raises(prx.PrError) as e:
            prx.bfs(dg, s)
        assert e.value.status == prx.PR_ERR_ARG
    short = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(prx.PrError) as e:
        prx.bfs(dg, 0, ws=short)
    assert e.value.status == prx.PR_ERR_WORKSPACE
    with pytest.raises(prx.PrError) as e:
        prx.wcc(dg, ws=short)
    assert e.value.status == prx.PR_ERR_WORKSPACE


@pytest.mark.slow
def test_rmat23_traversals(prx):
    """The headline graph at full size: BFS from vertex 0 (the largest
    out-degree of the unrelabelled R-MAT) and from a mid-range vertex, and
    the weak components, all bit-exact."""
    g = _cases.workload("rmat23")
    print(f"[rmat23] n={g.n} m={g.m}", flush=True)
    dg = _cases.gpu_graph(g)
    in_csr = prx.transpose(dg)
    for s in (0, 4_194_305):
        for ic in (None, in_csr):
            _check_bfs(prx, g, dg, s, in_csr=ic)
            print(f"[rmat23] bfs from {s} ok (in-edges: {ic is not None})", flush=True)
    for ic in (None, in_csr):
        _check_wcc(prx, g, dg, in_csr=ic)
        print(f"[rmat23] wcc ok (in-edges: {ic is not None})", flush=True)
